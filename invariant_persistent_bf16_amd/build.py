"""Build the HIP libraries (gfx950 only) in-tree: invariant_persistent_bf16_amd/libbi.so
and libbi_bench.so.

Every source is compiled to an object of its own (in parallel; the persistent
GEMM's tile shapes sit in separate sources for that reason), then each library
is linked from its objects.  Every kernel is compiled for gfx950 with -O3, no
fast-math, floating-point contraction off (each a*b+c in the source is two
roundings unless written as fmaf), and the packed-fp32 feature off.  The
compiler's intermediate files are kept in _build/ (-save-temps): the gfx950
assembly the library's code objects are assembled from,
_build/<source>-hip-amdgcn-amd-amdhsa-gfx950.s, is what
tests/test_asm_hazards_cpu.py checks.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
_OBJ = os.path.join(_HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
          "-ffp-contract=off", "-fno-fast-math",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]
LDFLAGS = [f"--offload-arch={ARCH}", "-fPIC", "-shared"]

GEMM16 = ["csrc/gemm16_256x256.hip", "csrc/gemm16_128x256.hip", "csrc/gemm16_256x128.hip",
          "csrc/gemm16_128x128.hip", "csrc/gemm16_192x256.hip"]
LIBS = {
    "libbi.so": ["csrc/api.hip"] + GEMM16,
    "libbi_bench.so": ["csrc/api.hip", "csrc/bench_api.hip", "csrc/gemm16_128x128_shared.hip"] + GEMM16,
}


def _obj(src):
    return os.path.join(_OBJ, os.path.basename(src).replace(".hip", ".o"))


def device_asm_path(src):
    """The gfx950 assembly of a library source, as the last build left it."""
    stem = os.path.basename(src)[:-len(".hip")]
    return os.path.join(_OBJ, f"{stem}-hip-amdgcn-amd-amdhsa-{ARCH}.s")


def device_asm_cmd(src, out_s):
    """Command that writes the gfx950 assembly of one source to out_s."""
    return [HIPCC] + CFLAGS + ["-I", os.path.join(_ROOT, "include"), "--offload-device-only", "-S",
                               os.path.join(_HERE, src), "-o", out_s]


def _compile(src, verbose):
    out = _obj(src)
    tmp = out + ".tmp.o"
    cmd = [HIPCC] + CFLAGS + ["-save-temps=obj", "-I", os.path.join(_ROOT, "include"), "-c",
                              os.path.join(_HERE, src), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _link(name, verbose):
    out = os.path.join(_HERE, name)
    tmp = out + ".tmp"
    cmd = [HIPCC] + LDFLAGS + [_obj(s) for s in LIBS[name]] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose=False):
    os.makedirs(_OBJ, exist_ok=True)
    srcs = sorted({s for v in LIBS.values() for s in v})
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda s: _compile(s, verbose), srcs))
    return [_link(n, verbose) for n in LIBS]


if __name__ == "__main__":
    build(verbose=True)

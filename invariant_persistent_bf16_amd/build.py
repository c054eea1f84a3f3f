"""Build the HIP library (gfx950 only) in-tree: invariant_persistent_bf16_amd/libbi.so.

One translation unit per library; every kernel is compiled for gfx950 with
-O3, no fast-math, floating-point contraction off (each a*b+c in the source
is two roundings unless written as fmaf), and the packed-fp32 feature off.
"""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
         "-ffp-contract=off", "-fno-fast-math",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]

LIBS = {
    "libbi.so": ["csrc/api.hip"],
    "libbi_bench.so": ["csrc/api.hip", "csrc/bench_api.hip"],
}


def build_one(name, verbose=False):
    srcs = [os.path.join(_HERE, s) for s in LIBS[name]]
    srcs = [s for s in srcs if os.path.exists(s)]
    if not srcs:
        return None
    out = os.path.join(_HERE, name)
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(_ROOT, "include")] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose=False):
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=len(LIBS)) as ex:
        outs = list(ex.map(lambda n: build_one(n, verbose), LIBS))
    return [o for o in outs if o]


if __name__ == "__main__":
    build(verbose=True)

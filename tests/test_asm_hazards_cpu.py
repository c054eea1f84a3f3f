"""No instruction touches the destination of a hand-written LDS read before
the wait that covers it (CPU only: reads the gfx950 assembly).

The persistent GEMM and the prefill kernel issue LDS fragment reads as inline
assembly.  The compiler takes such a read's destination registers as written
at issue and may hand them to another value at once, although the hardware
writes them only when the read returns.  In the GEMM the last K step's reads
of the next fragments are dead; before the fix, the epilogue copied
accumulators out of their AGPRs into exactly those registers ahead of the
loop's final wait, so a late read (two workgroups sharing a compute unit's
LDS) replaced accumulators with the zero-filled stage it was reading.

The check runs on the assembly that the library's code objects were
assembled from (kept by the build), or on a fresh compile when the build is
missing or older than the sources.  The same assembly's kernel metadata pins
the register budgets: no kernel spills, and the binary32 64x64-tile GEMM fits
two workgroups per compute unit.
"""
import glob
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import asm_hazards
from invariant_persistent_bf16_amd import build as hip_build

CSRC = os.path.join(os.path.dirname(hip_build.__file__), "csrc")


def _sources():
    return sorted({s for v in hip_build.LIBS.values() for s in v})


def _asm_texts():
    newest_src = max(os.path.getmtime(p) for p in glob.glob(os.path.join(CSRC, "*")))
    todo, texts = [], {}
    for src in _sources():
        p = hip_build.device_asm_path(src)
        if os.path.exists(p) and os.path.getmtime(p) >= newest_src:
            with open(p) as f:
                texts[src] = f.read()
        else:
            todo.append(src)
    if todo:
        with tempfile.TemporaryDirectory() as d:
            def one(src):
                out = os.path.join(d, os.path.basename(src) + ".s")
                subprocess.run(hip_build.device_asm_cmd(src, out), check=True,
                               stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
                with open(out) as f:
                    return src, f.read()
            with ThreadPoolExecutor(max_workers=min(len(todo), os.cpu_count() or 4)) as ex:
                texts.update(dict(ex.map(one, todo)))
    return texts


_BAD = """\
_Zbad:
	s_waitcnt lgkmcnt(0)
	;;#ASMSTART
	ds_read_b128 v[2:5], v40 offset:0
	;;#ASMEND
	v_mfma_f32_32x32x16_bf16 a[0:15], v[6:9], v[10:13], a[0:15]
	v_accvgpr_read_b32 v3, a7
	s_waitcnt vmcnt(0) lgkmcnt(0)
	global_store_dword v[20:21], v3, off
	s_endpgm
.Lfunc_end0:
"""

_GOOD = """\
_Zgood:
	;;#ASMSTART
	ds_read_b128 v[2:5], v40 offset:0
	;;#ASMEND
	v_accvgpr_read_b32 v30, a7
	s_cbranch_scc1 .LBB0_2
	v_add_u32_e32 v31, v30, v30
.LBB0_2:
	;;#ASMSTART
	s_waitcnt lgkmcnt(0)
	;;#ASMEND
	v_add_u32_e32 v3, v3, v30
	s_endpgm
.Lfunc_end1:
"""

_LOOP = """\
_Zloop:
.LBB2_1:
	v_mov_b32_e32 v4, 0
	;;#ASMSTART
	ds_read_b64_tr_b16 v[4:5], v40 offset:0
	;;#ASMEND
	s_cbranch_scc1 .LBB2_1
	s_waitcnt lgkmcnt(0)
	s_endpgm
.Lfunc_end2:
"""


def test_checker_flags_a_copy_into_a_pending_register():
    res = asm_hazards.check_file(_BAD)
    assert list(res) == ["_Zbad"]
    assert [h[2] for h in res["_Zbad"]] == [[3]]


def test_checker_accepts_waited_reads_and_follows_branches():
    assert asm_hazards.check_file(_GOOD) == {}


def test_checker_follows_loop_back_edges():
    # the read issued at the end of one iteration is still in flight when the
    # next iteration writes its register
    res = asm_hazards.check_file(_LOOP)
    assert [h[1] for h in res["_Zloop"]] == ["v_mov_b32_e32 v4, 0"]


@pytest.fixture(scope="module")
def texts():
    return _asm_texts()


def test_library_kernels_have_no_pending_register_hazard(texts):
    checked, found = 0, {}
    n_asm_reads = 0
    for src, txt in texts.items():
        fns = asm_hazards.functions(txt)
        checked += len(fns)
        n_asm_reads += txt.count("ds_read_b64_tr_b16") + txt.count("ds_read_b128")
        for name, hz in asm_hazards.check_file(txt).items():
            found[f"{src}:{name}"] = hz[:3]
    assert checked > 100, checked
    assert n_asm_reads > 1000, n_asm_reads
    assert not found, "\n".join(f"{k}: {v}" for k, v in list(found.items())[:10])


def _kernel_metadata(text):
    """(name, vgpr_count, vgpr_spill_count) of each kernel in an assembly file."""
    import re
    meta = text[text.find("amdhsa.kernels"):]
    out = []
    for block in meta.split("\n  - ")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        vg = re.search(r"\.vgpr_count:\s+(\d+)", block)
        sp = re.search(r"\.vgpr_spill_count:\s+(\d+)", block)
        if name and vg and sp:
            out.append((name.group(1), int(vg.group(1)), int(sp.group(1))))
    return out


def test_register_budgets():
    # No kernel of the library spills registers, and the binary32 64x64-tile
    # GEMM without a K tail fits 256 registers per lane, so that two of its
    # workgroups share a compute unit (its grid is four workgroups per CU;
    # at 332 registers it ran 24% slower at 4096 x 4096 x 1024).
    texts = _asm_texts()
    seen = 0
    for src, text in texts.items():
        for name, vgprs, spills in _kernel_metadata(text):
            seen += 1
            assert spills == 0, f"{name} spills {spills} registers"
            if name.startswith("_ZN2bi19gemm_f32_persistentIL") and "Lb0ELi32E" in name:
                assert vgprs <= 256, f"{name}: {vgprs} registers leave one workgroup per CU"
    assert seen > 50

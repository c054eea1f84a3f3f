"""bi_decode_attn_noalloc: the no-allocation variant of bi_decode_attn
(chunk triples in the library's static device scratch) gives bi_decode_attn's
bits, on two calls in a row, the second with a smaller input; a request whose
triples exceed the scratch is refused on the host before any launch.
"""
import ctypes

import pytest
import torch

import synth
from helpers import bitwise_equal

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
DEV = "cuda"
SCRATCH_BYTES = 32 << 20      # BI_DECODE_SCRATCH_BYTES in include/bi.h
BI_ERR_SCRATCH = -9


def _call(q, k, v, out):
    B, H, S, D = k.shape
    return bi.lib().bi_decode_attn_noalloc(B, H, S, D, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                           ctypes.c_float(0.125), bi.BI_BF16, bi._dt(out),
                                           torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("D", [64, 128])
def test_noalloc_matches_decode_twice_then_smaller(D):
    # first call: the decode workload's batch (B = 256 at D = 64); second
    # call: a smaller, ragged one
    shapes = [(256, 32, 8192), (3, 5, 5000)] if D == 64 else [(64, 32, 8192), (2, 7, 2049)]
    for i, (B, H, S) in enumerate(shapes):
        assert bi.bi_decode_attn_workspace_bytes(B, H, S, D) <= SCRATCH_BYTES
        print(f"noalloc decode call {i}: B={B} H={H} S={S} D={D}", flush=True)
        q = synth.randn((B, H, D), seed=40 + i, dtype=torch.bfloat16, device=DEV)
        k = synth.randn((B, H, S, D), seed=50 + i, dtype=torch.bfloat16, device=DEV)
        v = synth.randn((B, H, S, D), seed=60 + i, dtype=torch.bfloat16, device=DEV)
        for od in (torch.float32, torch.bfloat16):
            ref = bi.bi_decode_attn(q, k, v, 0.125, out_dtype=bi.BI_F32 if od == torch.float32 else bi.BI_BF16)
            out = torch.full((B, H, D), float("nan"), dtype=od, device=DEV)
            assert _call(q, k, v, out) == 0
            torch.cuda.synchronize()
            assert bitwise_equal(out, ref), f"call {i} ({od}) differs from bi_decode_attn"


def test_noalloc_refuses_more_than_the_scratch():
    B, H, S, D = 256, 32, 32768, 64       # 8 chunks per (b, h): 69 MB of triples
    assert bi.bi_decode_attn_workspace_bytes(B, H, S, D) > SCRATCH_BYTES
    q = torch.empty(16, dtype=torch.bfloat16, device=DEV)   # never read: refused first
    out = torch.empty(16, dtype=torch.float32, device=DEV)
    rc = bi.lib().bi_decode_attn_noalloc(B, H, S, D, q.data_ptr(), q.data_ptr(), q.data_ptr(), out.data_ptr(),
                                         ctypes.c_float(0.125), bi.BI_BF16, bi.BI_F32,
                                         torch.cuda.current_stream().cuda_stream)
    assert rc == BI_ERR_SCRATCH
    assert "scratch" in bi.status_string(rc)

"""GPU parity and invariance of bi_decode_attn (through the C ABI).

The decode workload: q [B, 32, 64], K, V [B, 32, 8192, 64] bf16 with fixed
2048-token chunks.  Request 0 must be bit for bit the same at B in
{1, 16, 64, 256}; request 0 and sampled requests match the unsplit fp64
oracle; ragged lengths, D = 128 and the closed forms (V = 1, q = 0) are
covered on small shapes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_bf16_rounding, assert_parity, bitwise_equal, to64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
DEV = "cuda"


def test_chunk_constant():
    assert bi.bi_decode_chunk_tokens() == 2048


@pytest.mark.parametrize("S", [1, 100, 2048, 2049, 5000, 8192])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_parity_ragged(S, D):
    B, H = 2, 3
    q = synth.randn((B, H, D), seed=S, dtype=torch.bfloat16)
    k = synth.randn((B, H, S, D), seed=S + 1, dtype=torch.bfloat16)
    v = synth.randn((B, H, S, D), seed=S + 2, dtype=torch.bfloat16)
    scale = 1.0 / np.sqrt(D)
    o32 = bi.bi_decode_attn(q.to(DEV), k.to(DEV), v.to(DEV), scale, out_dtype=bi.BI_F32)
    o16 = bi.bi_decode_attn(q.to(DEV), k.to(DEV), v.to(DEV), scale, out_dtype=bi.BI_BF16)
    torch.cuda.synchronize()
    ref = oracle.decode(q, k, v, float(np.float32(scale)))
    assert_parity(to64(o32), ref, f"decode S={S} D={D}")
    assert_bf16_rounding(o16, ref, f"decode bf16 S={S} D={D}")
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))


def test_decode_closed_forms():
    B, H, S, D = 2, 4, 8192, 64
    q = synth.randn((B, H, D), seed=40, dtype=torch.bfloat16).to(DEV)
    k = synth.randn((B, H, S, D), seed=41, dtype=torch.bfloat16).to(DEV)
    ones = torch.ones(B, H, S, D, dtype=torch.bfloat16, device=DEV)
    o = bi.bi_decode_attn(q, k, ones, 0.125)
    kc = torch.full((B, H, S, D), 0.5, dtype=torch.bfloat16, device=DEV)
    vt = (torch.arange(S, device=DEV) % 8).to(torch.bfloat16)[None, None, :, None].expand(B, H, S, D).contiguous()
    o2 = bi.bi_decode_attn(q, kc, vt, 0.125)
    vr = synth.randint((B, H, S, D), -8, 8, seed=42, dtype=torch.bfloat16)
    o3 = bi.bi_decode_attn(torch.zeros_like(q), k, vr.to(DEV), 0.125)
    torch.cuda.synchronize()
    assert torch.all(o == 1.0), "V = 1 must give exactly 1"
    assert torch.all(o2 == 3.5), "constant K, V[t] = t mod 8 must give exactly 3.5"
    assert np.array_equal(to64(o3), vr.double().mean(2).numpy()), "q = 0 must average V exactly"


def test_decode_request0_invariant_and_sampled_parity():
    qkv0 = synth.decode_shared()
    first = {}
    for B in (1, 16, 64, 256):
        q, k, v = synth.decode_batch(qkv0, B, device=DEV)
        o = bi.bi_decode_attn(q, k, v, 0.125)
        torch.cuda.synchronize()
        first[B] = o[0].clone()
        if B in (1, 256):
            reqs = [0] if B == 1 else [0, 1, 100, 255]
            qs, ks, vs = q[reqs].cpu(), k[reqs].cpu(), v[reqs].cpu()
            ref = oracle.decode(qs, ks, vs, 0.125)
            assert_parity(to64(o[reqs]), ref, f"decode B={B} sampled requests")
        del q, k, v, o
    for B in first:
        assert bitwise_equal(first[B], first[1]), f"request 0 differs at B={B}"


def test_decode_errors():
    q = torch.zeros(1, 1, 96, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 1, 16, 96, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(bi.BIError) as e:
        bi.bi_decode_attn(q, k, k, 0.1)
    assert e.value.status == -5
    q = torch.zeros(1, 1, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 1, 16, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(bi.BIError) as e:
        bi.bi_decode_attn(q, k, k, 0.1, workspace=torch.empty(1, device=DEV))
    assert e.value.status == -6

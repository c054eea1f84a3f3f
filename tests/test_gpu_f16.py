"""GPU parity and invariance of the binary16 (fp16) configuration of the
matmul family (through the C ABI): the pages fix one configuration per dtype
and list fp16 beside bf16.

Parity of bi_mm / bi_addmm / bi_bmm with fp16 operands against the fp64
oracle on ragged shapes in both B layouts; fp16 outputs equal the
round-to-nearest-even of the binary32 outputs bit for bit; row 0 is the same
at every batch size; a bmm slice equals the plain product; the SigLIP patch
embedding in fp16 keeps sample 0 bitwise across batch sizes.
"""
import pytest
import torch

import oracle
import synth
from helpers import assert_parity, bitwise_equal, to64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
DEV = "cuda"
F16 = torch.float16


def _rne16(c16, c32, what):
    assert torch.equal(c16.view(torch.int16), c32.to(F16).view(torch.int16)), f"{what}: not RNE of fp32"


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (70, 264, 512), (300, 520, 584), (257, 1000, 136)])
@pytest.mark.parametrize("b_layout", ["n_contig", "k_contig"])
def test_f16_addmm_parity_ragged(M, N, K, b_layout):
    A = synth.randn((M, K), seed=M + 11, dtype=F16)
    if b_layout == "n_contig":
        B = synth.randn((K, N), seed=N + 12, dtype=F16, scale=0.05)
    else:
        B = synth.randn((N, K), seed=N + 12, dtype=F16, scale=0.05).t()
    bias = synth.randn((N,), seed=K + 13, dtype=F16, scale=0.02)
    Ad, Bd, bd = A.to(DEV), B.to(DEV), bias.to(DEV)
    C32 = bi.bi_addmm(bd, Ad, Bd, out_dtype=bi.BI_F32)
    C16 = bi.bi_addmm(bd, Ad, Bd, out_dtype=bi.BI_F16)
    Cmm = bi.bi_mm(Ad, Bd, out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    assert C16.dtype == F16
    assert_parity(to64(C32), oracle.mm(A, B, bias), f"f16 addmm {M}x{N}x{K} {b_layout}")
    assert_parity(to64(Cmm), oracle.mm(A, B), f"f16 mm {M}x{N}x{K} {b_layout}")
    _rne16(C16, C32, "f16 addmm")


def test_f16_row0_invariant_and_bmm_slices():
    K, N = 4096, 1024
    W = synth.randn((K, N), seed=21, dtype=F16, scale=0.02).to(DEV)
    bias = synth.randn((N,), seed=22, dtype=F16, scale=0.02).to(DEV)
    X = synth.randn((513, K), seed=23, dtype=F16).to(DEV)
    outs = {M: bi.bi_addmm(bias, X[:M].contiguous(), W, out_dtype=bi.BI_F16) for M in (1, 8, 63, 64, 200, 513)}
    G = synth.randn((3, 200, K), seed=24, dtype=F16).to(DEV)
    Cb = bi.bi_bmm(G, W.expand(3, K, N).contiguous(), out_dtype=bi.BI_F32)
    C1 = bi.bi_mm(G[1].contiguous(), W, out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    for M, C in outs.items():
        assert bitwise_equal(C[:1], outs[1]), f"f16 row 0 differs at M={M}"
    assert bitwise_equal(Cb[1], C1), "bmm slice differs from mm"
    rows = [0, 100, 199]
    assert_parity(to64(C1[rows]), oracle.mm(G[1, rows].cpu(), W.cpu()), "f16 K=4096 sampled rows")


def test_f16_siglip_sample0_invariant():
    w, bias, x0 = synth.conv_shared()
    wd, bd = w.to(F16).to(DEV), bias.to(F16).to(DEV)
    first = None
    for B in (1, 4, 32):
        x = synth.conv_batch(x0, B).to(F16).to(DEV)
        y = bi.bi_conv2d(x, wd, bd, stride=(14, 14), out_dtype=bi.BI_F16)
        torch.cuda.synchronize()
        first = y[0].clone() if first is None else first
        assert bitwise_equal(y[0], first), f"f16 conv sample 0 differs at B={B}"
    ref = oracle.conv2d_direct(x0.to(F16), w.to(F16), bias.to(F16), (14, 14), samples=[0])
    y32 = bi.bi_conv2d(x0.to(F16).to(DEV), wd, bd, stride=(14, 14), out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    import numpy as np
    assert_parity(np.moveaxis(to64(y32), 1, -1), np.moveaxis(ref, 1, -1), "f16 siglip")

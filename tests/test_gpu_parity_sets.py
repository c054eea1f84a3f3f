"""Parity sets at the full workload sizes, in the launch configuration the
benchmark times, and the batch sweeps that cross every kernel the shape-only
choice can return.

Sampled parity (binary32 outputs against the fp64 oracle on the same inputs,
relative L2 <= 1e-5 and per-row max-abs <= 1e-4 * ||row||_2; bfloat16 outputs
as roundings of values within that band):
  * addmm X [M, 4096] @ W [4096, 14336] + bias at M = 2048 and 8192: row 0
    plus 63 seeded random rows;
  * decode q [B, 32, 64], K, V [B, 32, 8192, 64] at B = 64 and 256: request 0
    plus 63 seeded random requests (all of them at B = 64);
  * the SigLIP patch convolution at 32 images: image 0 plus 15 seeded images;
  * attention at B = 32 (256 slices of 1024 x 1024 x 128), stage by stage on
    the GPU's own intermediates: S = Q K^T on 8 slices, the softmax of the
    GPU's S rows, and O = P V from the GPU's bfloat16 P ("Batch-Invariant
    Kernel Design: Conv2d and Attention BMM", section "Kernel 2: Attention
    BMM"; the products run on the same 256x256 and 256x128 tiles as in the
    benchmark, asserted below).
Every comparison also yields the figures of the VLA page's tracer
(helpers.comparison_record).

Batch sweeps (row 0 / image 0 bit for bit against batch 1): addmm at
M in {1, 63, 64, 200, 384, 576, 768, 1152, 2048, 8192} and the convolution at
B in {1, 2, 4, 16, 32, 48}, with the kernel each size selects asserted, so
the sweep crosses the small-tile kernel (32 and 64 rows) and every persistent
tile shape (128x128, 128x256, 192x256, 256x256).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (assert_bf16_is_rne_of, assert_bf16_rounding, assert_parity, bitwise_equal,
                     comparison_record, to64)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
    from invariant_persistent_bf16_amd import bi_bench
DEV = "cuda"
SCALE = float(torch.tensor(1 / math.sqrt(128), dtype=torch.float32))


def _sample(n_total, n_random, seed):
    """Index 0 plus n_random distinct seeded indices from 1 .. n_total-1."""
    g = torch.Generator().manual_seed(seed)
    rest = (torch.randperm(n_total - 1, generator=g)[:n_random] + 1).tolist()
    return [0] + sorted(rest)


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


# -------------------------------------------------------------------- addmm
@pytest.mark.parametrize("M", [2048, 8192])
def test_addmm_row0_plus_63_rows(M):
    W, bias, x0 = synth.addmm_shared()
    Wd, bd = W.to(DEV), bias.to(DEV)
    X = synth.addmm_batch(x0, M, device=DEV)
    print(f"addmm M={M}: kernel choice {bi_bench.gemm_tile_rows(1, M, 14336, 4096)}", flush=True)
    C32 = bi.bi_addmm(bd, X, Wd, out_dtype=bi.BI_F32)
    C16 = bi.bi_addmm(bd, X, Wd, out_dtype=bi.BI_BF16)
    torch.cuda.synchronize()
    rows = _sample(M, 63, seed=7000 + M)
    ref = oracle.mm(X[rows].cpu(), W, bias)
    got = to64(C32[rows])
    assert_parity(got, ref, f"addmm M={M} rows")
    assert_bf16_rounding(C16[rows], ref, f"addmm M={M} bf16 rows")
    assert_bf16_is_rne_of(C16, C32, f"addmm M={M}")
    rec = comparison_record(got, ref, f"addmm M={M}: 64 rows vs oracle")
    print(rec, flush=True)


def test_addmm_row0_sweep_crosses_every_kernel():
    W, bias, x0 = synth.addmm_shared()
    Wd, bd = W.to(DEV), bias.to(DEV)
    Ms = (1, 63, 64, 200, 384, 576, 768, 1152, 2048, 8192)
    picks = {M: bi_bench.gemm_tile_rows(1, M, 14336, 4096) for M in Ms}
    print(f"addmm kernel choice by M: {picks}", flush=True)
    if _cus() == 256:
        # 32 / 64: small-tile kernel rows; 3: 128x128, 1: 128x256, 4: 192x256, 0: 256x256
        assert picks == {1: 32, 63: 64, 64: 64, 200: 3, 384: 1, 576: 4, 768: 4, 1152: 1, 2048: 0, 8192: 0}
    row0 = {}
    for M in Ms:
        X = synth.addmm_batch(x0, M, device=DEV)
        C = bi.bi_addmm(bd, X, Wd, out_dtype=bi.BI_F32)
        torch.cuda.synchronize()
        row0[M] = C[0].clone()
        del X, C
    for M in Ms:
        assert bitwise_equal(row0[M], row0[1]), f"row 0 differs at M={M} (kernel {picks[M]})"
    rec = comparison_record(np.stack([to64(row0[M]) for M in Ms]),
                            np.stack([to64(row0[1])] * len(Ms)), "addmm row 0, M sweep vs M=1")
    assert rec["max_abs_diff"] == 0.0


# ------------------------------------------------------------------- decode
@pytest.mark.parametrize("B", [64, 256])
def test_decode_request0_plus_63_requests(B):
    qkv0 = synth.decode_shared()
    q, k, v = synth.decode_batch(qkv0, B, device=DEV)
    o32 = bi.bi_decode_attn(q, k, v, 0.125)
    o16 = bi.bi_decode_attn(q, k, v, 0.125, out_dtype=bi.BI_BF16)
    torch.cuda.synchronize()
    reqs = _sample(B, 63, seed=8000 + B)
    assert len(reqs) == 64
    ref = oracle.decode(q[reqs].cpu(), k[reqs].cpu(), v[reqs].cpu(), 0.125)
    got = to64(o32[reqs])
    assert_parity(got, ref, f"decode B={B} requests")
    assert_bf16_rounding(o16[reqs], ref, f"decode bf16 B={B}")
    assert_bf16_is_rne_of(o16, o32, f"decode B={B}")
    print(comparison_record(got, ref, f"decode B={B}: 64 requests vs oracle"), flush=True)


# --------------------------------------------------------------------- conv
def _chlast(y):
    return np.moveaxis(np.asarray(y), 1, -1)


def test_conv_b32_sixteen_images():
    w, bias, x0 = synth.conv_shared()
    x = synth.conv_batch(x0, 32, device=DEV)
    y32 = bi.bi_conv2d(x, w.to(DEV), bias.to(DEV), stride=(14, 14), out_dtype=bi.BI_F32)
    y16 = bi.bi_conv2d(x, w.to(DEV), bias.to(DEV), stride=(14, 14), out_dtype=bi.BI_BF16)
    torch.cuda.synchronize()
    imgs = _sample(32, 15, seed=9032)
    ref = _chlast(oracle.conv2d_direct(x[imgs].cpu(), w, bias, stride=(14, 14)))
    got = _chlast(to64(y32[imgs]))
    assert_parity(got, ref, "conv B=32 images")
    assert_bf16_rounding(torch.from_numpy(_chlast(to64(y16[imgs]))).to(torch.bfloat16), ref, "conv bf16 B=32")
    assert_bf16_is_rne_of(y16, y32, "conv B=32")
    print(comparison_record(got, ref, "conv B=32: 16 images vs oracle"), flush=True)


def test_conv_image0_sweep_crosses_every_kernel():
    w, bias, x0 = synth.conv_shared()
    wd, bd = w.to(DEV), bias.to(DEV)
    Bs = (1, 2, 4, 16, 32, 48)
    picks = {B: bi_bench.gemm_tile_rows(B, 1152, 256, 592) for B in Bs}
    print(f"conv GEMM kernel choice by B: {picks}", flush=True)
    if _cus() == 256:
        assert picks == {1: 32, 2: 64, 4: 3, 16: 1, 32: 4, 48: 0}
    first = {}
    for B in Bs:
        x = synth.conv_batch(x0, B, device=DEV)
        y = bi.bi_conv2d(x, wd, bd, stride=(14, 14), out_dtype=bi.BI_F32)
        torch.cuda.synchronize()
        first[B] = y[0].clone()
        del x, y
    for B in Bs:
        assert bitwise_equal(first[B], first[1]), f"image 0 differs at B={B} (kernel {picks[B]})"


# ---------------------------------------------------------------- attention
def test_attention_b32_stages_on_gpu_intermediates():
    B, H, T, D = 32, 8, 1024, 128
    G = B * H
    Q, K, V = synth.attn_batch(synth.attn_shared(), B, device=DEV)
    if _cus() == 256:
        assert bi_bench.gemm_tile_rows(G, T, T, D) == 0       # S = Q K^T: 256x256 tiles
        assert bi_bench.gemm_tile_rows(G, T, D, T) == 2       # O = P V: 256x128 tiles
    S = torch.empty(G, T, T, dtype=torch.float32, device=DEV)
    P = torch.empty(G, T, T, dtype=torch.bfloat16, device=DEV)
    O = bi.attention(Q, K, V, SCALE, S_buf=S, P_buf=P)
    P32 = bi.bi_softmax_rows(S.view(G * T, T), SCALE, out_dtype=bi.BI_F32).view(G, T, T)
    torch.cuda.synchronize()
    sl = _sample(G, 7, seed=9100)
    Qs, Ks, Vs = Q[sl].cpu(), K[sl].cpu(), V[sl].cpu()
    # stage 1: S = Q K^T
    ref_s = oracle.bmm(Qs, Ks.transpose(1, 2))
    assert_parity(to64(S[sl]), ref_s, "attention B=32 stage 1 (S)")
    print(comparison_record(to64(S[sl]), ref_s, "attention B=32 S, 8 slices"), flush=True)
    # stage 2: the softmax of the GPU's own S rows
    S_gpu = S[sl].cpu().reshape(-1, T)
    ref_p = oracle.softmax_rows(S_gpu, SCALE)
    assert_parity(to64(P32[sl]).reshape(-1, T), ref_p, "attention B=32 stage 2 (P, fp32)")
    assert_bf16_rounding(P[sl].reshape(-1, T), ref_p, "attention B=32 stage 2 (P, bf16)")
    assert_bf16_is_rne_of(P[sl], P32[sl], "attention B=32 P")
    print(comparison_record(to64(P32[sl]).reshape(len(sl), -1), ref_p.reshape(len(sl), -1),
                            "attention B=32 P (fp32) on the GPU's S, 8 slices"), flush=True)
    # stage 3: O = P V on the GPU's own bfloat16 P
    ref_o = oracle.bmm(P[sl].cpu(), Vs)
    assert_parity(to64(O[sl]), ref_o, "attention B=32 stage 3 (O)")
    print(comparison_record(to64(O[sl]), ref_o, "attention B=32 O on the GPU's P, 8 slices"), flush=True)

"""GPU parity and invariance of the attention path (bi_bmm, bi_softmax_rows, bi_bmm).

Each stage is checked against the oracle on its own seeded inputs
(S = Q K^T; P = softmax(scale S); O = P V), and the whole path end to end.
Slice 0 (all 8 heads of batch element 0) must be bit for bit the same at
B = 1 and B = 32.  The end-to-end comparison feeds the oracle's own bfloat16
rounding of its fp64 P into its second product; the GPU rounds its binary32
P, so elements that sit within binary32 error of a bfloat16 rounding boundary
may round the other way: that stage is gated by a bound derived from one
bfloat16 unit in the last place of P (see DESIGN), the stages by 1e-5.
The one-kernel probabilities (bi_attention_probs: scores in LDS, never in
memory) must give the two-stage P bit for bit, on ragged and strided shapes
and on the whole B = 32 workload, and then the same O.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_bf16_rounding, assert_parity, bitwise_equal, rel_l2, to64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
DEV = "cuda"
SCALE = float(torch.tensor(1 / math.sqrt(128), dtype=torch.float32))


def test_stage1_qk_parity():
    Q, K, V = synth.attn_batch(synth.attn_shared(), 1)
    S = bi.bi_bmm(Q.to(DEV), K.to(DEV).transpose(1, 2), out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    ref = oracle.bmm(Q[:2], K[:2].transpose(1, 2))
    assert_parity(to64(S[:2]), ref, "S = Q K^T")


@pytest.mark.parametrize("cols", [1, 100, 1024, 1500, 4096, 5000])
def test_stage2_softmax_parity(cols):
    rows = 64
    S = synth.randn((rows, cols), seed=cols, scale=math.sqrt(128.0))
    P32 = bi.bi_softmax_rows(S.to(DEV), SCALE, out_dtype=bi.BI_F32)
    P16 = bi.bi_softmax_rows(S.to(DEV), SCALE, out_dtype=bi.BI_BF16)
    torch.cuda.synchronize()
    ref = oracle.softmax_rows(S, SCALE)
    assert_parity(to64(P32), ref, f"softmax cols={cols}")
    assert_bf16_rounding(P16, ref, f"softmax bf16 cols={cols}")
    assert torch.equal(P16.view(torch.int16), P32.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("cols", [1020, 1024, 1023, 4096, 4097, 6000])
def test_stage2_softmax_vector_and_element_paths_same_bits(cols):
    # Rows read with 16-byte loads (aligned) and with element loads (the same
    # rows one float off alignment) share one reduction tree: same bits.
    rows = 40
    S = synth.randn((rows, cols), seed=cols + 11, scale=3.0)
    buf = torch.empty(rows * cols + 4, dtype=torch.float32, device=DEV)
    aligned = buf[:rows * cols].view(rows, cols)
    shifted = buf[1:1 + rows * cols].view(rows, cols)
    outs = []
    for view in (aligned, shifted):
        view.copy_(S.to(DEV))
        outs.append((bi.bi_softmax_rows(view, SCALE, out_dtype=bi.BI_F32),
                     bi.bi_softmax_rows(view, SCALE, out_dtype=bi.BI_BF16)))
        torch.cuda.synchronize()
    assert bitwise_equal(outs[0][0], outs[1][0]), "binary32 P depends on the load path"
    assert bitwise_equal(outs[0][1], outs[1][1]), "bfloat16 P depends on the load path"
    assert_parity(to64(outs[0][0]), oracle.softmax_rows(S, SCALE), f"softmax cols={cols}")


def test_stage2_softmax_strided_rows_and_row_invariance():
    S = synth.randn((300, 1100), seed=5, scale=4.0)
    Sd = S.to(DEV)
    P = bi.bi_softmax_rows(Sd[:, :1024], SCALE, out_dtype=bi.BI_F32)
    P1 = bi.bi_softmax_rows(Sd[:1, :1024], SCALE, out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    assert bitwise_equal(P[:1], P1)
    assert_parity(to64(P), oracle.softmax_rows(S[:, :1024], SCALE), "softmax strided")


def test_stage3_pv_parity():
    # P: nonnegative rows summing to about one, rounded to bf16.
    G, T, D = 4, 1024, 128
    u = synth.uniform((G, T, T), seed=6)
    P = (u / u.sum(-1, keepdim=True)).to(torch.bfloat16)
    V = synth.randn((G, T, D), seed=7, dtype=torch.bfloat16)
    O = bi.bi_bmm(P.to(DEV), V.to(DEV), out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    assert_parity(to64(O), oracle.bmm(P, V), "O = P V")


def test_zero_query_gives_mean_of_v_exactly():
    G, T, D = 2, 1024, 128
    Q = torch.zeros(G, T, D, dtype=torch.bfloat16, device=DEV)
    K = synth.randn((G, T, D), seed=8, dtype=torch.bfloat16).to(DEV)
    V = synth.randint((G, T, D), -8, 8, seed=9, dtype=torch.bfloat16)
    O = bi.attention(Q, K, V.to(DEV), SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(to64(O), oracle.attention(Q.cpu(), K.cpu(), V, SCALE, p_bf16=True))


def test_slice0_invariant_B1_vs_B32_and_end_to_end():
    qkv0 = synth.attn_shared()
    outs = {}
    for B in (1, 32):
        Q, K, V = synth.attn_batch(qkv0, B, device=DEV)
        S_buf = torch.empty(8 * B, 1024, 1024, dtype=torch.float32, device=DEV)
        O = bi.attention(Q, K, V, SCALE, S_buf=S_buf)
        torch.cuda.synchronize()
        outs[B] = (O[:8].clone(), S_buf[:8].clone())
        del Q, K, V, S_buf, O
    assert bitwise_equal(outs[1][1], outs[32][1]), "S of batch element 0 differs"
    assert bitwise_equal(outs[1][0], outs[32][0]), "O of batch element 0 differs"
    Q, K, V = (t.reshape(-1, 1024, 128) for t in qkv0)
    ref = oracle.attention(Q[:2], K[:2], V[:2], SCALE, p_bf16=True)
    got = to64(outs[1][0][:2])
    e = rel_l2(got, ref)
    # One bfloat16 rounding step of P (2^-8 relative) on every element is the
    # worst case; observed flips are rare, so the error sits far below it.
    assert e <= 2.0 ** -8, f"end-to-end rel-L2 {e}"
    assert_parity(got, ref, "attention end-to-end", rel=1e-3, row=1e-2)


def _two_stage_probs(Q, K, scale):
    G, T, D = Q.shape
    S = bi.bi_bmm(Q, K.transpose(1, 2), out_dtype=bi.BI_F32)
    return bi.bi_softmax_rows(S.view(G * T, -1), scale, out_dtype=bi.BI_BF16).view(G, T, -1)


@pytest.mark.parametrize("G,T,Tk,D", [(4, 1024, 1024, 128), (3, 100, 256, 64), (2, 33, 512, 128),
                                      (5, 1, 768, 64), (300, 64, 256, 128), (1, 1000, 1024, 128)])
def test_fused_probs_same_bits_as_two_stages(G, T, Tk, D):
    # bi_attention_probs runs the bmm's MFMA chain and the softmax's reduction
    # tree without writing S: P must equal bi_bmm -> bi_softmax_rows bit for
    # bit; ragged query blocks (T % 32), one query row, more slices than CUs,
    # and one slice split over many workgroups.
    Q = synth.randn((G, T, D), seed=G + T, dtype=torch.bfloat16).to(DEV)
    K = synth.randn((G, Tk, D), seed=Tk + D, dtype=torch.bfloat16).to(DEV)
    for scale in (float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32)), 0.37):
        P = bi.bi_attention_probs(Q, K, scale)
        ref = _two_stage_probs(Q, K, scale)
        torch.cuda.synchronize()
        assert bitwise_equal(P, ref), f"fused P differs (scale {scale})"


def test_fused_probs_strided_views_and_errors():
    G, T, Tk, D = 3, 70, 512, 64
    Qw = synth.randn((G, T, 2 * D), seed=51, dtype=torch.bfloat16).to(DEV)
    Kw = synth.randn((G, Tk, 3 * D), seed=52, dtype=torch.bfloat16).to(DEV)
    Q, K = Qw[:, :, D:], Kw[:, :, :D]           # row strides 2D and 3D
    Pw = torch.empty(G, T, Tk + 64, dtype=torch.bfloat16, device=DEV)
    P = bi.bi_attention_probs(Q, K, 0.125, out=Pw[:, :, :Tk])
    ref = _two_stage_probs(Q.contiguous(), K.contiguous(), 0.125)
    torch.cuda.synchronize()
    assert bitwise_equal(P, ref)
    with pytest.raises(RuntimeError, match="BI_ERR_UNSUPPORTED"):
        bi.bi_attention_probs(Q[:, :, :32], K[:, :, :32], 0.125)          # D = 32
    with pytest.raises(RuntimeError, match="BI_ERR_UNSUPPORTED"):
        bi.bi_attention_probs(Q, K[:, :300], 0.125)                        # Tk = 300


def test_fused_attention_bench_config_same_bits():
    # The B = 32 workload (256 slices of 1024 x 1024 x 128): every P and O bit
    # equal to the three-launch path's.
    Q, K, V = synth.attn_batch(synth.attn_shared(), 32, device=DEV)
    S_buf = torch.empty(256, 1024, 1024, dtype=torch.float32, device=DEV)
    P_ref = torch.empty(256, 1024, 1024, dtype=torch.bfloat16, device=DEV)
    O_ref = bi.attention(Q, K, V, SCALE, S_buf=S_buf, P_buf=P_ref)
    del S_buf
    P = torch.empty_like(P_ref)
    O = bi.attention(Q, K, V, SCALE, P_buf=P)
    torch.cuda.synchronize()
    assert bitwise_equal(P, P_ref), "fused P differs at the bench config"
    assert bitwise_equal(O, O_ref), "O differs at the bench config"

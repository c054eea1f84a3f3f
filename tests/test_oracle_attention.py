"""Pins of the oracle's softmax, attention and decode attention (CPU only).

Closed forms (rows summing to one, uniform weights for a zero query, constant
V), torch's float64 softmax and attention as independent library routines,
the identity between one-chunk flash decoding and unsplit attention, and the
booleans the deterministic-inference handbook prints for its two binary32
experiments (split-K GEMM, flash decoding).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ softmax
def test_softmax_rows_sum_to_one_and_match_torch():
    S = synth.randn((37, 300), seed=1, scale=6.0)
    scale = float(torch.tensor(1 / math.sqrt(128), dtype=torch.float32))
    P = oracle.softmax_rows(S, scale)
    assert np.all(np.abs(P.sum(1) - 1.0) <= 1e-12)
    ref = torch.softmax(S.double() * scale, dim=1).numpy()
    np.testing.assert_allclose(P, ref, rtol=1e-13, atol=1e-16)


def test_softmax_shift_invariance_and_strided_rows():
    base = synth.randint((5, 64), -40, 40, seed=2) / 8      # multiples of 1/8: +3 is exact
    wide = torch.zeros(5, 80)
    wide[:, :64] = base
    P1 = oracle.softmax_rows(wide[:, :64], 1.0)
    P2 = oracle.softmax_rows(base + 3.0, 1.0)
    assert np.array_equal(P1, P2)


def test_softmax_equal_scores_are_uniform():
    P = oracle.softmax_rows(torch.full((3, 1024), 0.75), 0.5)
    assert np.all(P == 2.0 ** -10)


# ---------------------------------------------------------------- attention
def test_attention_matches_torch_float64():
    G, T, D = 3, 20, 8
    Q, K, V = (synth.randn((G, T, D), seed=s, dtype=torch.bfloat16) for s in (3, 4, 5))
    scale = 1 / math.sqrt(D)
    O = oracle.attention(Q, K, V, scale)
    q, k, v = Q.double(), K.double(), V.double()
    ref = torch.softmax(q @ k.transpose(1, 2).contiguous() * scale, dim=-1) @ v
    np.testing.assert_allclose(O, ref.numpy(), rtol=1e-12, atol=1e-13)
    ref2 = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    np.testing.assert_allclose(O, ref2.numpy(), rtol=1e-12, atol=1e-13)


def test_attention_zero_query_averages_v():
    G, T, D = 2, 1024, 4
    Q = torch.zeros(G, T, D, dtype=torch.bfloat16)
    K = synth.randn((G, T, D), seed=6, dtype=torch.bfloat16)
    V = synth.randint((G, T, D), -8, 8, seed=7, dtype=torch.bfloat16)
    O = oracle.attention(Q, K, V, 0.3, p_bf16=True)   # P = 2^-10 exactly, also in bf16
    mean = V.double().mean(1, keepdim=True).expand(G, T, D).numpy()
    assert np.array_equal(O, mean)


def test_attention_bf16_p_is_rounded_softmax():
    G, T, D = 1, 16, 4
    Q, K = (synth.randn((G, T, D), seed=s, dtype=torch.bfloat16) for s in (8, 9))
    V = torch.eye(T, dtype=torch.bfloat16)[None, :, :D].contiguous()  # O[:, d] picks P[:, d]
    scale = 0.5
    P = torch.softmax(Q.double() @ K.double().transpose(1, 2).contiguous() * scale, -1)[0].numpy()
    O = oracle.attention(Q, K, V, scale, p_bf16=True)[0]
    assert np.array_equal(O, oracle.bf16_rne_array(P[:, :D]))


def test_attention_slice_subset():
    Q, K, V = (synth.randn((4, 8, 4), seed=s) for s in (10, 11, 12))
    full = oracle.attention(Q, K, V, 0.5)
    assert np.array_equal(oracle.attention(Q, K, V, 0.5, slices=[2, 0]), full[[2, 0]])


# ------------------------------------------------------------------- decode
def _decode_case(B=2, H=3, S=300, D=16, seed=20, dtype=torch.bfloat16):
    q = synth.randn((B, H, D), seed=seed, dtype=dtype)
    k = synth.randn((B, H, S, D), seed=seed + 1, dtype=dtype)
    v = synth.randn((B, H, S, D), seed=seed + 2, dtype=dtype)
    return q, k, v


def test_decode_matches_torch_float64():
    q, k, v = _decode_case()
    scale = 0.25
    out = oracle.decode(q, k, v, scale)
    qd, kd, vd = q.double(), k.double(), v.double()
    s = torch.einsum("bhd,bhsd->bhs", qd, kd) * scale
    ref = torch.einsum("bhs,bhsd->bhd", torch.softmax(s, -1), vd)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_one_chunk_merge_equals_unsplit_bitwise():
    q, k, v = _decode_case()
    unsplit = oracle.decode(q, k, v, 0.25)
    for chunk in (300, 512, 2048):
        assert np.array_equal(oracle.decode_chunked(q, k, v, 0.25, chunk=chunk), unsplit)


@pytest.mark.parametrize("chunk", [64, 100, 128, 299])
def test_chunked_merge_equals_unsplit(chunk):
    q, k, v = _decode_case()
    np.testing.assert_allclose(oracle.decode_chunked(q, k, v, 0.25, chunk=chunk),
                               oracle.decode(q, k, v, 0.25), rtol=1e-13, atol=1e-14)


def test_chunk_triples_follow_definition():
    q, k, v = _decode_case(B=1, H=1, S=100, D=4)
    out, trip = oracle.decode_chunked(q, k, v, 0.5, chunk=32, triples=True)
    assert trip.shape == (1, 1, 4, 6)
    s = (k.double()[0, 0] @ q.double()[0, 0]) * 0.5
    for c in range(4):
        sc = s[32 * c: 32 * c + 32]
        m = sc.max()
        p = torch.exp(sc - m)
        assert trip[0, 0, c, 0] == m.item()
        np.testing.assert_allclose(trip[0, 0, c, 1], p.sum().item(), rtol=1e-14)
        np.testing.assert_allclose(trip[0, 0, c, 2:], (p @ v.double()[0, 0, 32 * c: 32 * c + 32]).numpy(),
                                   rtol=1e-13, atol=1e-15)


def test_decode_closed_forms():
    B, H, S, D = 1, 2, 8192, 64
    q = synth.randn((B, H, D), seed=30, dtype=torch.bfloat16)
    k = synth.randn((B, H, S, D), seed=31, dtype=torch.bfloat16)
    ones = torch.ones(B, H, S, D, dtype=torch.bfloat16)
    assert np.all(oracle.decode_chunked(q, k, ones, 0.125) == 1.0)
    kc = torch.full((B, H, S, D), 0.5, dtype=torch.bfloat16)
    vt = (torch.arange(S) % 8).to(torch.bfloat16)[None, None, :, None].expand(B, H, S, D).contiguous()
    assert np.all(oracle.decode_chunked(q, kc, vt, 0.125) == 3.5)
    q0 = torch.zeros(B, H, D, dtype=torch.bfloat16)
    vr = synth.randint((B, H, S, D), -8, 8, seed=32, dtype=torch.bfloat16)
    mean = vr.double().mean(2).numpy()     # sums of small integers: exact
    assert np.array_equal(oracle.decode_chunked(q0, k, vr, 0.125), mean)


def test_decode_request_subset():
    q, k, v = _decode_case(B=3)
    full = oracle.decode_chunked(q, k, v, 0.25, chunk=128)
    assert np.array_equal(oracle.decode_chunked(q, k, v, 0.25, chunk=128, reqs=[2]), full[[2]])


# ---------------------------------------------- the handbook's experiments
def test_handbook_splitk_pattern():
    g = json.load(open(os.path.join(GOLDEN, "handbook_splitk_gemm.json")))
    K, N = g["setup"]["K"], g["setup"]["N"]
    W, X = synth.mm_inputs(Ms=g["batches"], K=K, N=N, seed=g["setup"]["seed"])
    mine = X[g["batches"][0]][:1]
    for invariant, key in ((False, "row0_equals_alone_by_batch"), (True, "row0_equals_alone_fixed")):
        def splits(M):
            return 1 if invariant or M >= 64 else 4
        alone = oracle.sim_splitk_gemm_f32(mine, W, splits(1))[0]
        got = [bool(torch.equal(oracle.sim_splitk_gemm_f32(X[M], W, splits(M))[0], alone))
               for M in g["batches"]]
        assert got == g[key]


def test_handbook_decode_pattern():
    g = json.load(open(os.path.join(GOLDEN, "handbook_decode_splits.json")))
    D, S = g["setup"]["D"], g["setup"]["S"]
    gen = torch.Generator().manual_seed(g["setup"]["seed"])
    q = torch.randn(D, generator=gen)
    K = torch.randn(S, D, generator=gen)
    V = torch.randn(S, D, generator=gen)
    scale = 1 / D ** 0.5

    def by_load(b, sms=132):
        return max(1, min(64, sms // b))

    assert [by_load(b) for b in g["batches"]] == g["splits_by_load"]
    ref = oracle.sim_decode_splits_f32(q, K, V, scale, by_load(1))
    got = [bool(torch.equal(oracle.sim_decode_splits_f32(q, K, V, scale, by_load(b)), ref))
           for b in g["batches"]]
    assert got == g["equal_to_batch1_by_load"]
    nfix = -(-S // 2048)
    assert nfix == g["splits_fixed"]
    fixed = [oracle.sim_decode_splits_f32(q, K, V, scale, nfix) for _ in g["batches"]]
    assert all(torch.equal(f, fixed[0]) for f in fixed) == g["fixed_all_equal"]
    unsplit = torch.softmax(K @ q / D ** 0.5, 0) @ V
    assert torch.allclose(fixed[0], unsplit, atol=g["fixed_allclose_unsplit_atol"]) == g["fixed_allclose_unsplit"]
    # The fixed-chunk fp64 oracle agrees with the binary32 simulation to binary32 accuracy.
    o64 = oracle.decode_chunked(q.to(torch.float32)[None, None], K[None, None], V[None, None], scale)[0, 0]
    np.testing.assert_allclose(fixed[0].double().numpy(), o64, rtol=0, atol=1e-5)

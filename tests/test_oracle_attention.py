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
# Both experiments are driven by the fixture: its setup holds the sizes, the
# seed and the parameters of the two split rules, and its booleans are the
# ones the page prints.  The binary32 simulations are the oracle's C code.
def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _row0_pattern(X, W, x0, batches, split_rule):
    """For each batch size M: does row 0 of the split-K product of X[M] equal
    the product of x0 alone, each with the split count split_rule gives?"""
    alone = oracle.sim_splitk_gemm_f32(x0, W, split_rule(1))[0].numpy()
    return [bool(np.array_equal(oracle.sim_splitk_gemm_f32(X[m], W, split_rule(m))[0].numpy(), alone))
            for m in batches]


def test_handbook_splitk_pattern():
    g = _golden("handbook_splitk_gemm.json")
    st = g["setup"]
    W, X = synth.mm_inputs(Ms=g["batches"], K=st["K"], N=st["N"], seed=st["seed"])
    x0 = X[g["batches"][0]][:1]
    tuned = st["tuned"]
    rules = {
        "row0_equals_alone_by_batch": lambda m: tuned["splits"] if m < tuned["below_batch"] else 1,
        "row0_equals_alone_fixed": lambda m: st["fixed_splits"],
    }
    for key, rule in rules.items():
        assert _row0_pattern(X, W, x0, g["batches"], rule) == g[key], key


def test_handbook_decode_pattern():
    g = _golden("handbook_decode_splits.json")
    st = g["setup"]
    D, S = st["D"], st["S"]
    gen = torch.Generator().manual_seed(st["seed"])
    q, K, V = (torch.randn(shape, generator=gen) for shape in ((D,), (S, D), (S, D)))
    scale = 1 / D ** 0.5
    by_load = st["by_load"]
    parts = [min(by_load["max_parts"], max(1, by_load["units"] // b)) for b in g["batches"]]
    assert parts == g["splits_by_load"]
    results = {n: oracle.sim_decode_splits_f32(q, K, V, scale, n).numpy() for n in sorted(set(parts))}
    assert [bool(np.array_equal(results[n], results[parts[0]])) for n in parts] == g["equal_to_batch1_by_load"]
    # fixed-length chunks: the part count is a function of S only
    n_fixed = -(-S // st["fixed_chunk"])
    assert n_fixed == g["splits_fixed"]
    fixed = [oracle.sim_decode_splits_f32(q, K, V, scale, n_fixed).numpy() for _ in g["batches"]]
    assert (len({f.tobytes() for f in fixed}) == 1) == g["fixed_all_equal"]
    # against unsplit attention (the fp64 oracle, one query)
    unsplit = oracle.decode(q[None, None], K[None, None], V[None, None], scale)[0, 0]
    close = bool(np.max(np.abs(fixed[0].astype(np.float64) - unsplit)) <= g["fixed_allclose_unsplit_atol"])
    assert close == g["fixed_allclose_unsplit"]
    # the fixed-chunk fp64 oracle agrees with the binary32 simulation to binary32 accuracy
    o64 = oracle.decode_chunked(q[None, None], K[None, None], V[None, None], scale)[0, 0]
    np.testing.assert_allclose(fixed[0].astype(np.float64), o64, rtol=0, atol=1e-5)

"""Pins of the oracle's matrix products (CPU only).

The oracle is checked against things other than itself: closed forms
(identity, all-ones), exact integer arithmetic in Python, exact rational
arithmetic, numpy's float64 matmul, and torch's binary32 -> bfloat16 rounding.
Non-square shapes with distinct dimensions make a transposed operand or a
swapped index fail.
"""
import fractions
import itertools

import numpy as np
import pytest
import torch

import oracle
import synth


def _bits(t):
    return t.view(torch.int16).numpy().astype(np.uint16)


def test_widen_bf16_bit_patterns():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,
             0x0080: 2.0 ** -126, 0x3E80: 0.25, 0x8000: -0.0, 0x4049: 3.140625}
    raw = torch.tensor(list(cases.keys()), dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    for i, v in enumerate(cases.values()):
        assert oracle.widen(raw, i) == v


def test_bf16_rne_matches_torch_rounding_of_binary32():
    # For values exactly representable in binary32 a single RNE to bfloat16 from
    # double equals torch's binary32 -> bfloat16 RNE.
    x = synth.randn((20000,), seed=7) * torch.logspace(-30, 30, 20000)
    ref = x.to(torch.bfloat16).double().numpy()
    got = oracle.bf16_rne_array(x.double().numpy())
    assert np.array_equal(got, ref)


def test_bf16_rne_ties_and_specials():
    assert oracle.bf16_rne(1.0 + 2 ** -8) == 1.0               # tie -> even (1.0)
    assert oracle.bf16_rne(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6  # tie -> even (odd ulp rounds up)
    assert oracle.bf16_rne(1.0 + 2 ** -8 + 2 ** -30) == 1.0 + 2 ** -7
    assert oracle.bf16_rne(-(1.0 + 2 ** -8 + 2 ** -30)) == -(1.0 + 2 ** -7)
    assert oracle.bf16_rne(2.0 ** -134) == 0.0                  # half the subnormal quantum, tie -> 0
    assert oracle.bf16_rne(1.5 * 2.0 ** -133) == 2.0 ** -132
    assert oracle.bf16_rne(2.0 ** 128) == float("inf")
    assert oracle.bf16_rne((2 - 2 ** -7) * 2.0 ** 127) == (2 - 2 ** -7) * 2.0 ** 127
    # Double rounding through binary32 would give 1 + 2^-7 here; one rounding gives 1.
    assert oracle.bf16_rne(1.0 + 2 ** -8 - 2 ** -40) == 1.0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_identity_and_ones(dtype):
    M, K, N = 7, 24, 5
    A = synth.randn((M, K), seed=1, dtype=dtype)
    eye = torch.eye(K, dtype=dtype)
    assert np.array_equal(oracle.mm(A, eye), A.double().numpy())
    ones_a = torch.ones(M, K, dtype=dtype)
    ones_b = torch.ones(K, N, dtype=dtype)
    bias = synth.randn((N,), seed=2, dtype=dtype)
    assert np.array_equal(oracle.mm(ones_a, ones_b), np.full((M, N), float(K)))
    assert np.array_equal(oracle.mm(ones_a, ones_b, bias), float(K) + bias.double().numpy()[None, :].repeat(M, 0))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("b_layout", ["n_contig", "k_contig"])
def test_small_integers_exact(dtype, b_layout):
    M, K, N = 5, 13, 6
    A = synth.randint((M, K), -4, 4, seed=3, dtype=dtype)
    if b_layout == "n_contig":
        B = synth.randint((K, N), -4, 4, seed=4, dtype=dtype)
    else:
        B = synth.randint((N, K), -4, 4, seed=4, dtype=dtype).t()   # K-contiguous view
    bias = synth.randint((N,), -9, 9, seed=5, dtype=dtype)
    a = [[int(v) for v in row] for row in A.tolist()]
    b = [[int(v) for v in row] for row in B.tolist()]
    exact = [[sum(a[i][k] * b[k][j] for k in range(K)) + int(bias[j]) for j in range(N)] for i in range(M)]
    assert np.array_equal(oracle.mm(A, B, bias), np.array(exact, dtype=np.float64))


def test_random_bf16_against_exact_rationals():
    M, K, N = 3, 40, 4
    A = synth.randn((M, K), seed=11, dtype=torch.bfloat16)
    B = synth.randn((K, N), seed=12, dtype=torch.bfloat16)
    got = oracle.mm(A, B)
    for i, j in itertools.product(range(M), range(N)):
        ex = sum(fractions.Fraction(float(A[i, k])) * fractions.Fraction(float(B[k, j])) for k in range(K))
        mag = sum(abs(float(A[i, k]) * float(B[k, j])) for k in range(K))
        assert abs(got[i, j] - float(ex)) <= K * 2 ** -52 * mag


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 17, 9), (33, 70, 65), (64, 128, 19)])
def test_against_numpy_float64(shape):
    M, K, N = shape
    A = synth.randn((M, K), seed=21, dtype=torch.bfloat16)
    B = synth.randn((K, N), seed=22, dtype=torch.bfloat16)
    bias = synth.randn((N,), seed=23, dtype=torch.bfloat16)
    ref = A.double().numpy() @ B.double().numpy() + bias.double().numpy()
    np.testing.assert_allclose(oracle.mm(A, B, bias), ref, rtol=1e-13, atol=1e-13)


def test_strided_views_and_row_subset():
    M, K, N = 20, 16, 12
    big = synth.randn((M, 2 * K), seed=31)
    A = big[:, ::2]                      # non-unit K stride
    B = synth.randn((N, K), seed=32).t()  # K-contiguous
    full = oracle.mm(A, B)
    np.testing.assert_allclose(full, A.double().numpy() @ B.double().numpy(), rtol=1e-13, atol=1e-13)
    rows = [19, 0, 7]
    assert np.array_equal(oracle.mm(A, B, rows=rows), full[rows])


def test_bmm_is_per_slice_mm():
    G, M, K, N = 4, 6, 10, 7
    A = synth.randn((G, M, K), seed=41, dtype=torch.bfloat16)
    B = synth.randn((G, N, K), seed=42, dtype=torch.bfloat16).transpose(1, 2)
    out = oracle.bmm(A, B)
    ref = np.matmul(A.double().numpy(), B.double().numpy())
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)
    for g in range(G):
        assert np.array_equal(out[g], oracle.mm(A[g], B[g]))
    assert np.array_equal(oracle.bmm(A, B, slices=[3, 1]), out[[3, 1]])


def test_bias_added_after_sum():
    # A bias much larger than the products: adding it first would absorb the
    # small terms in binary64; adding it last keeps them.
    K = 4
    A = torch.full((1, K), 2.0 ** -30, dtype=torch.float32)
    B = torch.ones(K, 1, dtype=torch.float32)
    bias = torch.tensor([2.0 ** 24], dtype=torch.float32)
    got = oracle.mm(A, B, bias)[0, 0]
    assert got == 2.0 ** 24 + 4 * 2.0 ** -30


def test_thread_count_changes_no_result():
    # the benchmark times the oracle on one core and on all of them
    A = synth.randn((37, 300), seed=91, dtype=torch.bfloat16)
    B = synth.randn((300, 50), seed=92, dtype=torch.bfloat16)
    n = oracle.set_threads()
    try:
        oracle.set_threads(1)
        one = oracle.mm(A, B)
        oracle.set_threads(max(n, 4))
        many = oracle.mm(A, B)
    finally:
        oracle.set_threads(n)
    assert np.array_equal(one, many)

"""Pins of the oracle's binary16 (fp16) inputs (CPU only).

The widening of every one of the 65536 fp16 bit patterns equals numpy's
float16 -> float64 conversion (an independent implementation); an fp16 matrix
product of small integers equals exact integer arithmetic, and of random fp16
values equals numpy float64 on the widened operands; the fp16 batched product
slices equal per-slice products.
"""
import numpy as np
import torch

import oracle


def test_f16_widening_all_bit_patterns():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    t = bits.view(torch.float16)
    got = np.array([oracle.widen(t, i) for i in range(65536)])
    ref = bits.numpy().view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_f16_mm_small_integers_exact():
    g = torch.Generator().manual_seed(0)
    A = torch.randint(-20, 21, (37, 64), generator=g).to(torch.float16)
    B = torch.randint(-20, 21, (64, 29), generator=g).to(torch.float16)
    exact = (A.long() @ B.long()).numpy().astype(np.float64)
    assert np.array_equal(oracle.mm(A, B), exact)


def test_f16_mm_and_bmm_random():
    g = torch.Generator().manual_seed(1)
    A = torch.randn(3, 33, 80, generator=g).to(torch.float16)
    B = torch.randn(3, 80, 47, generator=g).to(torch.float16)
    ref = np.matmul(A.numpy().astype(np.float64), B.numpy().astype(np.float64))
    got = oracle.bmm(A, B)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.abs(ref).max()
    assert np.array_equal(got[1], oracle.mm(A[1], B[1]))

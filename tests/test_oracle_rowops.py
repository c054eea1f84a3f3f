"""Pins of the oracle's row operations: RMSNorm, log-softmax, row mean (CPU only).

Each is pinned by closed forms a dropped term, a wrong divisor or a sign slip
would break, by invariances, and by torch's float64 library routines
(`torch.nn.functional.rms_norm`, `torch.log_softmax`, `torch.mean`) as
independent implementations.  The RMSNorm identity mean(y^2) =
ms / (ms + eps) (w = 1) restates the pages' worked example in "Beyond Matrix
Multiplication" ("RMS of normalized ... close to 1") as an exact relation.
"""
import math

import numpy as np
import torch

import oracle
import synth


# ------------------------------------------------------------------ RMSNorm
def test_rms_norm_matches_torch_float64():
    x = synth.randn((7, 300), seed=1)
    w = synth.randn((300,), seed=2)
    got = oracle.rms_norm(x, w, 1e-6)
    ref = torch.nn.functional.rms_norm(x.double(), (300,), w.double(), 1e-6).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_rms_norm_pages_example_rms_identity():
    # The pages' example: batch 2, seq 4, hidden 8, weight ones; with w = 1,
    # mean(y^2) = ms / (ms + eps) exactly, ms = mean(x^2), i.e. RMS close to 1.
    x = synth.randn((2 * 4, 8), seed=3)
    for eps in (1e-6, 0.5):
        y = oracle.rms_norm(x, torch.ones(8), eps)
        ms = (x.double() ** 2).mean(1).numpy()
        np.testing.assert_allclose((y ** 2).mean(1), ms / (ms + eps), rtol=1e-14)


def test_rms_norm_closed_forms():
    # Rows of +-2^k: y = sign * w exactly (eps = 0); a one-hot row c*e_j gives
    # y_j = sign(c) * sqrt(cols) * w_j (mean over cols, not a sum) and zeros elsewhere.
    cols = 64
    w = synth.randn((cols,), seed=4)
    x = torch.full((3, cols), 0.25)
    x[1] = -8.0
    x[2, ::2] = -0.25
    y = oracle.rms_norm(x, w, 0.0)
    sign = np.sign(x.double().numpy())
    assert np.array_equal(y, sign * w.double().numpy())
    oh = torch.zeros(1, cols)
    oh[0, 5] = -3.0
    y = oracle.rms_norm(oh, w, 0.0)[0]
    assert math.isclose(y[5], -math.sqrt(cols) * float(w[5]), rel_tol=1e-15)
    assert np.count_nonzero(y) == 1


def test_rms_norm_scale_invariance_and_bf16_widening():
    x = synth.randn((5, 129), seed=5, dtype=torch.bfloat16)
    w = synth.randn((129,), seed=6, dtype=torch.bfloat16)
    y1 = oracle.rms_norm(x, w, 0.0)
    y2 = oracle.rms_norm((x.float() * 4.0).to(torch.bfloat16), w, 0.0)   # exact scaling
    np.testing.assert_allclose(y1, y2, rtol=1e-15, atol=0)
    ref = torch.nn.functional.rms_norm(x.double(), (129,), w.double(), 0.0).numpy()
    np.testing.assert_allclose(y1, ref, rtol=1e-13)


def test_rms_norm_strided_rows():
    wide = synth.randn((6, 100), seed=7)
    w = synth.randn((64,), seed=8)
    assert np.array_equal(oracle.rms_norm(wide[:, :64], w, 1e-6),
                          oracle.rms_norm(wide[:, :64].contiguous(), w, 1e-6))


# -------------------------------------------------------------- log-softmax
def test_log_softmax_matches_torch_float64():
    x = synth.randn((9, 1000), seed=9, scale=5.0)
    got = oracle.log_softmax_rows(x)
    ref = torch.log_softmax(x.double(), dim=1).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_log_softmax_normalised_shift_invariant_constant_rows():
    x = synth.randn((4, 333), seed=10, scale=3.0)
    y = oracle.log_softmax_rows(x)
    np.testing.assert_allclose(np.exp(y).sum(1), 1.0, rtol=1e-14)
    y2 = oracle.log_softmax_rows(x + 2.0)   # x + 2 is not exact in fp32 everywhere: compare loosely
    np.testing.assert_allclose(y, y2, atol=1e-5)
    c = oracle.log_softmax_rows(torch.full((2, 1024), -7.5))
    assert np.all(c == -math.log(1024.0))


def test_log_softmax_two_element_closed_form():
    a, b = 1.5, -2.25
    y = oracle.log_softmax_rows(torch.tensor([[a, b]]))[0]
    # log(sum) near 1 loses a few ulps against log1p: 1e-13, not exact.
    assert math.isclose(y[0], -math.log1p(math.exp(b - a)), rel_tol=1e-13)
    assert math.isclose(y[1], (b - a) - math.log1p(math.exp(b - a)), rel_tol=1e-13)


# -------------------------------------------------------------------- mean
def test_mean_rows_closed_forms_and_torch():
    n = 1001
    x = torch.arange(n, dtype=torch.float32).repeat(3, 1)
    assert np.all(oracle.mean_rows(x) == (n - 1) / 2)
    xi = synth.randint((5, 777), -100, 100, seed=11, dtype=torch.bfloat16)
    exact = xi.double().sum(1).numpy() / 777
    assert np.array_equal(oracle.mean_rows(xi), exact)
    xr = synth.randn((4, 4096), seed=12)
    np.testing.assert_allclose(oracle.mean_rows(xr), torch.mean(xr.double(), 1).numpy(), rtol=1e-12, atol=1e-15)


def test_mean_rows_strided():
    wide = synth.randn((3, 50), seed=13)
    assert np.array_equal(oracle.mean_rows(wide[:, 10:40]), oracle.mean_rows(wide[:, 10:40].contiguous()))

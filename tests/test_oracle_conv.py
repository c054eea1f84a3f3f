"""Pins of the oracle's convolution (CPU only).

Closed forms (all-ones, one-hot kernels), the SigLIP geometry printed on the
pages, an independent patchify formulation, the oracle's second (unfold)
route, and torch's float64 CPU convolution with stride, padding, dilation
and groups.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_siglip_geometry_matches_page():
    g = json.load(open(os.path.join(GOLDEN, "siglip_patch_embed.json")))
    oh = oracle.conv_out(g["image"][0], g["kernel"][0], g["stride"][0], g["padding"][0], 1)
    ow = oracle.conv_out(g["image"][1], g["kernel"][1], g["stride"][1], g["padding"][1], 1)
    assert [oh, ow] == g["grid"] and oh * ow == g["tokens"]
    assert g["in_channels"] * g["kernel"][0] * g["kernel"][1] == g["reduction_length"]


def test_ones_give_reduction_length_plus_bias():
    x = torch.ones(2, 3, 28, 28, dtype=torch.bfloat16)
    w = torch.ones(6, 3, 14, 14, dtype=torch.bfloat16)
    bias = synth.randn((6,), seed=1, dtype=torch.bfloat16)
    y = oracle.conv2d_direct(x, w, bias, stride=(14, 14))
    ref = 588.0 + bias.double().numpy()[None, :, None, None]
    assert np.array_equal(y, np.broadcast_to(ref, (2, 6, 2, 2)))


def test_one_hot_kernel_picks_strided_pixels():
    C, S = 3, 14
    x = synth.uniform((2, C, 56, 56), seed=2, lo=-1, hi=1, dtype=torch.bfloat16)
    w = torch.zeros(C, C, S, S, dtype=torch.bfloat16)
    for c in range(C):
        w[c, c, 0, 0] = 1.0
    y = oracle.conv2d_direct(x, w, None, stride=(S, S))
    assert np.array_equal(y, x[:, :, ::S, ::S].double().numpy())


def test_patchify_formulation_siglip_shape():
    # With stride == kernel and no padding the unfold is a permutation: cut the
    # image into 14x14 patches, flatten each as (c, kh, kw) and multiply.
    w, bias, x0 = synth.conv_shared(Cout=32)
    x = x0
    y = oracle.conv2d_direct(x, w, bias, stride=(14, 14))
    p = x.double().reshape(1, 3, 16, 14, 16, 14).permute(0, 2, 4, 1, 3, 5).reshape(1, 256, 588)
    ref = (p @ w.double().reshape(32, 588).t() + bias.double()).permute(0, 2, 1).reshape(1, 32, 16, 16)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


CASES = [
    # (N, Cin, H, W, Cout, Kh, Kw, stride, padding, dilation, groups)
    (2, 3, 11, 13, 4, 3, 3, (1, 1), (0, 0), (1, 1), 1),
    (1, 4, 9, 10, 6, 3, 2, (2, 1), (1, 2), (1, 1), 2),
    (2, 6, 12, 12, 6, 3, 3, (1, 2), (2, 1), (2, 2), 3),
    (1, 2, 8, 7, 3, 5, 1, (3, 1), (2, 0), (1, 3), 1),
    (3, 3, 28, 28, 5, 14, 14, (14, 14), (0, 0), (1, 1), 1),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_direct_vs_unfold_vs_torch(case, dtype):
    N, Cin, H, W, Cout, Kh, Kw, st, pd, dl, gr = case
    x = synth.randn((N, Cin, H, W), seed=10, dtype=dtype)
    w = synth.randn((Cout, Cin // gr, Kh, Kw), seed=11, dtype=dtype)
    b = synth.randn((Cout,), seed=12, dtype=dtype)
    y = oracle.conv2d_direct(x, w, b, st, pd, dl, gr)
    u = oracle.conv2d_unfold(x, w, b, st, pd, dl, gr)
    ref = F.conv2d(x.double(), w.double(), b.double(), st, pd, dl, gr).numpy()
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, u, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_sample_subset():
    x = synth.randn((4, 2, 9, 9), seed=20)
    w = synth.randn((3, 2, 3, 3), seed=21)
    full = oracle.conv2d_direct(x, w, None, (2, 2), (1, 1))
    assert np.array_equal(oracle.conv2d_direct(x, w, None, (2, 2), (1, 1), samples=[3, 0]), full[[3, 0]])


def test_small_integers_exact():
    x = synth.randint((1, 3, 28, 28), -4, 4, seed=30, dtype=torch.bfloat16)
    w = synth.randint((4, 3, 14, 14), -4, 4, seed=31, dtype=torch.bfloat16)
    y = oracle.conv2d_direct(x, w, None, stride=(14, 14))
    ref = F.conv2d(x.to(torch.int64).double(), w.double(), None, (14, 14))  # exact: |sum| < 2^53
    xi = x.to(torch.int64)
    wi = w.to(torch.int64)
    exact = torch.einsum("nchw,ochw->no", xi.reshape(1, 3, 2, 14, 2, 14).permute(0, 2, 4, 1, 3, 5)
                         .reshape(4, 3, 14, 14), wi).t().reshape(1, 4, 2, 2)
    assert np.array_equal(y, exact.double().numpy())
    assert np.array_equal(y, ref.numpy())

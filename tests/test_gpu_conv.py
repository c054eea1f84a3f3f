"""GPU parity and invariance of bi_conv2d (through the C ABI).

The SigLIP patch embedding (3 -> 1152 channels, 14x14 kernel, stride 14, 224x224
images): sample 0 bit for bit the same at B in {1, 2, 4, 8, 16, 32} (the
batch sweep of the VLA page), sampled outputs against the direct seven-loop
oracle; general stride / padding / dilation / groups cases against the
oracle (16-bit cases with no padding, one group and even kernel width,
column stride and width take the specialised unfolds, by 16-byte pieces or,
where input rows come in whole pieces, by rows of locations, the SigLIP
shape among them); the all-ones closed form and integer inputs exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_bf16_is_rne_of, assert_bf16_rounding, assert_parity, bitwise_equal, to64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
DEV = "cuda"


def _chlast(y):
    # rows of the convolution: the Cout outputs of one location
    return np.moveaxis(np.asarray(y), 1, -1)


def test_siglip_sample0_invariant_and_parity():
    w, bias, x0 = synth.conv_shared()
    wd, bd = w.to(DEV), bias.to(DEV)
    first16, first32 = {}, {}
    for B in (1, 2, 4, 8, 16, 32):
        x = synth.conv_batch(x0, B)
        xd = x.to(DEV)
        y32 = bi.bi_conv2d(xd, wd, bd, stride=(14, 14), out_dtype=bi.BI_F32)
        y16 = bi.bi_conv2d(xd, wd, bd, stride=(14, 14), out_dtype=bi.BI_BF16)
        torch.cuda.synchronize()
        assert y32.shape == (B, 1152, 16, 16)
        first32[B], first16[B] = y32[0].clone(), y16[0].clone()
        if B in (1, 32):
            samples = [0] if B == 1 else [0, 17, 31]
            ref = oracle.conv2d_direct(x, w, bias, stride=(14, 14), samples=samples)
            assert_parity(_chlast(to64(y32[samples])), _chlast(ref), f"conv B={B}")
            assert_bf16_rounding(torch.from_numpy(_chlast(to64(y16[samples]))).to(torch.bfloat16),
                                 _chlast(ref), f"conv bf16 B={B}")
            assert_bf16_is_rne_of(y16, y32, f"conv B={B}")
    for B in first32:
        assert bitwise_equal(first32[B], first32[1]), f"sample 0 (fp32 out) differs at B={B}"
        assert bitwise_equal(first16[B], first16[1]), f"sample 0 (bf16 out) differs at B={B}"


def test_siglip_ones_closed_form():
    x = torch.ones(2, 3, 224, 224, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(1152, 3, 14, 14, dtype=torch.bfloat16, device=DEV)
    bias = torch.full((1152,), 0.25, dtype=torch.bfloat16, device=DEV)
    y = bi.bi_conv2d(x, w, bias, stride=(14, 14), out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    assert torch.all(y == 588.25)


def test_siglip_integer_inputs_bitwise():
    x = synth.randint((2, 3, 224, 224), -4, 4, seed=3, dtype=torch.bfloat16)
    w = synth.randint((128, 3, 14, 14), -4, 4, seed=4, dtype=torch.bfloat16)
    y = bi.bi_conv2d(x.to(DEV), w.to(DEV), None, stride=(14, 14), out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    assert np.array_equal(to64(y), oracle.conv2d_direct(x, w, None, stride=(14, 14)))


CASES = [
    # (N, Cin, H, W, Cout, Kh, Kw, stride, padding, dilation, groups)
    (2, 3, 17, 19, 40, 3, 3, (1, 1), (1, 1), (1, 1), 1),
    (3, 4, 20, 21, 24, 3, 2, (2, 1), (1, 2), (1, 1), 2),
    (2, 6, 24, 24, 12, 3, 3, (1, 2), (2, 1), (2, 2), 3),
    (1, 8, 9, 33, 300, 5, 1, (3, 1), (2, 0), (1, 3), 1),
    (2, 16, 12, 12, 16, 3, 3, (1, 1), (1, 1), (1, 1), 16),
    # Non-overlapping patches (stride = kernel, no padding), with groups and
    # an input height that leaves rows unused; then rows of 20 elements.
    (2, 4, 35, 48, 20, 4, 8, (4, 8), (0, 0), (1, 1), 2),
    (1, 3, 20, 20, 8, 5, 5, (5, 5), (0, 0), (1, 1), 1),
    (2, 5, 27, 24, 16, 4, 6, (4, 6), (0, 0), (1, 1), 1),
    # The specialised unfold for 16-bit data with even Kw, column stride and
    # W, no padding, one group: overlapping windows, a zero-padded K
    # (Kg = 12 -> 16) and locations per row that are not a power of two.
    (2, 3, 11, 14, 24, 3, 4, (1, 2), (0, 0), (1, 1), 1),
    (3, 3, 16, 18, 10, 2, 2, (2, 2), (0, 0), (1, 1), 1),
    (2, 2, 13, 22, 9, 3, 4, (2, 4), (0, 0), (1, 1), 1),
    # Row blocks in whole 16-byte pieces (W = 16, 40): one workgroup per row
    # of locations; overlapping rows with unused input rows and a padded K,
    # then non-overlapping patches; then blocks too large for its LDS budget
    # (48 channels x 4 rows x 136), which fall back to the piecewise unfold.
    (2, 3, 20, 16, 12, 3, 4, (2, 2), (0, 0), (1, 1), 1),
    (3, 5, 24, 40, 16, 6, 8, (6, 8), (0, 0), (1, 1), 1),
    (1, 48, 8, 136, 8, 4, 4, (4, 4), (0, 0), (1, 1), 1),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_general_conv_parity(case, dtype):
    N, Cin, H, W, Cout, Kh, Kw, st, pd, dl, gr = case
    x = synth.randn((N, Cin, H, W), seed=30, dtype=dtype)
    w = synth.randn((Cout, Cin // gr, Kh, Kw), seed=31, dtype=dtype, scale=0.1)
    b = synth.randn((Cout,), seed=32, dtype=dtype, scale=0.1)
    y = bi.bi_conv2d(x.to(DEV), w.to(DEV), b.to(DEV), st, pd, dl, gr, out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    ref = oracle.conv2d_direct(x, w, b, st, pd, dl, gr)
    assert_parity(_chlast(to64(y)), _chlast(ref), f"conv {case} {dtype}")
    # Sample 0 alone gives the same bits.
    y0 = bi.bi_conv2d(x[:1].to(DEV), w.to(DEV), b.to(DEV), st, pd, dl, gr, out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    assert bitwise_equal(y0[0], y[0])


def test_conv_workspace_errors():
    x = torch.zeros(1, 3, 28, 28, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(4, 3, 14, 14, dtype=torch.bfloat16, device=DEV)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(bi.BIError) as e:
        bi.bi_conv2d(x, w, None, stride=(14, 14), workspace=small)
    assert e.value.status == -6

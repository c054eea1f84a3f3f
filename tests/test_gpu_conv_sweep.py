"""Seeded random sweep of bi_conv2d geometries (through the C ABI).

Each case draws the batch, channels, input size, kernel, stride, padding,
dilation, groups, operand dtype and bias from its seed; a third of the cases
are patch-like (stride equal to the kernel, no padding, one group, widths in
whole 16-byte pieces), so the specialised unfolds are drawn as well as the
general one.  The binary32 output is compared with the direct seven-loop
oracle on every output, and sample 0 computed alone gives the same bits as in
the batch ("Batch-Invariant Kernel Design: Conv2d and Attention BMM", section
"The two correctness tests").
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_parity, bitwise_equal, to64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
DEV = "cuda"
CASES = 36


def _geometry(seed):
    rng = np.random.default_rng(5000 + seed)
    r = lambda lo, hi: int(rng.integers(lo, hi + 1))
    dtype = [torch.bfloat16, torch.bfloat16, torch.float16, torch.float32][r(0, 3)]
    if seed % 3 == 0:   # patch-like
        Kh, Kw = r(1, 8), 2 * r(1, 4)
        g = dict(N=r(1, 3), Cin=r(1, 6), Kh=Kh, Kw=Kw, stride=(Kh, Kw), padding=(0, 0), dilation=(1, 1),
                 groups=1, Cout=r(1, 48))
        g["H"] = Kh * r(1, 5) + r(0, Kh - 1)
        g["W"] = 8 * r(1, 8) if Kw <= 8 else Kw * r(1, 4)
    else:
        groups = int(rng.choice([1, 1, 2, 3]))
        g = dict(N=r(1, 3), Cin=groups * r(1, 4), Kh=r(1, 5), Kw=r(1, 5), stride=(r(1, 3), r(1, 3)),
                 padding=(r(0, 2), r(0, 2)), dilation=(r(1, 2), r(1, 2)), groups=groups,
                 Cout=groups * r(1, 12))
        g["H"] = r(1, 24)
        g["W"] = r(1, 24)
    ext_h = g["dilation"][0] * (g["Kh"] - 1) + 1
    ext_w = g["dilation"][1] * (g["Kw"] - 1) + 1
    # at least one output location in each direction
    g["H"] = max(g["H"], ext_h - 2 * g["padding"][0])
    g["W"] = max(g["W"], ext_w - 2 * g["padding"][1])
    if seed % 3 == 0 and g["W"] % 8 and Kw <= 8:
        g["W"] += 8 - g["W"] % 8
    g["bias"] = bool(rng.integers(0, 4))
    return g, dtype


@pytest.mark.parametrize("seed", range(CASES))
def test_random_geometry_parity_and_sample0(seed):
    g, dtype = _geometry(seed)
    name = f"seed {seed}: {g} {dtype}"
    print(name, flush=True)
    st, pd, dl, gr = g["stride"], g["padding"], g["dilation"], g["groups"]
    x = synth.randn((g["N"], g["Cin"], g["H"], g["W"]), seed=seed, dtype=dtype)
    w = synth.randn((g["Cout"], g["Cin"] // gr, g["Kh"], g["Kw"]), seed=seed + 1, dtype=dtype, scale=0.1)
    b = synth.randn((g["Cout"],), seed=seed + 2, dtype=dtype, scale=0.1) if g["bias"] else None
    xd, wd = x.to(DEV), w.to(DEV)
    bd = None if b is None else b.to(DEV)
    y = bi.bi_conv2d(xd, wd, bd, st, pd, dl, gr, out_dtype=bi.BI_F32)
    y0 = bi.bi_conv2d(xd[:1], wd, bd, st, pd, dl, gr, out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    ref = oracle.conv2d_direct(x, w, b, st, pd, dl, gr)
    assert y.shape == ref.shape, name
    got = np.moveaxis(to64(y), 1, -1)
    assert_parity(got, np.moveaxis(ref, 1, -1), name)
    assert bitwise_equal(y0[0], y[0]), f"{name}: sample 0 alone differs"

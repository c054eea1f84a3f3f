"""GPU parity and invariance of the row operations (bi_rms_norm,
bi_log_softmax_rows, bi_mean_rows), through the C ABI.

Each is compared with the fp64 oracle on the same seeded inputs across every
regime of the row length (one wave per row up to 4096 columns, one workgroup
per row up to 16384, re-reading beyond), with ragged column counts, both input
dtypes, and at the LLM shapes the bench times on sampled rows.  Invariance:
row 0 alone gives the same bits as row 0 of a large batch, and with more rows
than the resident workgroups hold (RMSNorm's waves then loop over rows) every
sampled row, the last included, equals that row alone; aligned rows (vector
loads) and the same rows one element off alignment (element loads) give the
same bits; bfloat16 output is RNE of the binary32 output.  Closed forms:
RMSNorm of rows of +-2^k with eps = 0 is +-w exactly; the mean of small
integers is the correctly rounded exact mean.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_bf16_is_rne_of, assert_parity, bitwise_equal, to64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
DEV = "cuda"
COLS = [1, 3, 100, 1023, 1024, 1500, 4096, 4097, 10000, 16384, 20000]


def _sync():
    torch.cuda.synchronize()


@pytest.mark.parametrize("cols", COLS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rms_norm_parity(cols, dtype):
    rows = 24
    x = synth.randn((rows, cols), seed=cols, dtype=dtype)
    w = synth.randn((cols,), seed=cols + 1, dtype=dtype)
    y32 = bi.bi_rms_norm(x.to(DEV), w.to(DEV), 1e-6, out_dtype=bi.BI_F32)
    y16 = bi.bi_rms_norm(x.to(DEV), w.to(DEV), 1e-6, out_dtype=bi.BI_BF16)
    _sync()
    assert_parity(to64(y32), oracle.rms_norm(x, w, 1e-6), f"rms_norm cols={cols} {dtype}")
    assert_bf16_is_rne_of(y16, y32, "rms_norm bf16 out")


@pytest.mark.parametrize("cols", COLS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_log_softmax_parity(cols, dtype):
    rows = 24
    x = synth.randn((rows, cols), seed=cols + 2, dtype=dtype, scale=4.0)
    y32 = bi.bi_log_softmax_rows(x.to(DEV), out_dtype=bi.BI_F32)
    y16 = bi.bi_log_softmax_rows(x.to(DEV), out_dtype=bi.BI_BF16)
    _sync()
    assert_parity(to64(y32), oracle.log_softmax_rows(x), f"log_softmax cols={cols} {dtype}")
    assert_bf16_is_rne_of(y16, y32, "log_softmax bf16 out")


@pytest.mark.parametrize("cols", COLS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_mean_rows_parity(cols, dtype):
    rows = 40
    x = synth.randn((rows, cols), seed=cols + 3, dtype=dtype) + 0.5   # nonzero means
    y = bi.bi_mean_rows(x.to(DEV))
    y16 = bi.bi_mean_rows(x.to(DEV), out_dtype=bi.BI_BF16)
    _sync()
    # One output per row: each output is its own comparison row, so its bound
    # is 1e-4 of its own magnitude.
    assert_parity(to64(y)[:, None], oracle.mean_rows(x)[:, None], f"mean cols={cols} {dtype}")
    assert_bf16_is_rne_of(y16, y, "mean bf16 out")


@pytest.mark.parametrize("cols", [1000, 4096, 10000, 20000])
def test_row_zero_invariant_and_load_paths_agree(cols):
    rows = 300
    x = synth.randn((rows, cols), seed=cols + 4, scale=2.0)
    w = synth.randn((cols,), seed=cols + 5)
    xd, wd = x.to(DEV), w.to(DEV)
    buf = torch.empty(rows * cols + 4, dtype=torch.float32, device=DEV)
    shifted = buf[1:1 + rows * cols].view(rows, cols)   # one element off 16-byte alignment
    shifted.copy_(xd)
    for f in (lambda t: bi.bi_rms_norm(t, wd, 1e-6), bi.bi_log_softmax_rows, bi.bi_mean_rows):
        full, one, mis = f(xd), f(xd[:1]), f(shifted)
        _sync()
        assert bitwise_equal(full[:1], one), "row 0 depends on the number of rows"
        assert bitwise_equal(full, mis), "vector and element loads disagree"


def test_closed_forms():
    cols = 4096
    w = synth.randn((cols,), seed=6, dtype=torch.bfloat16)
    x = torch.full((3, cols), 0.25, dtype=torch.bfloat16)
    x[1] = -8.0
    x[2, ::2] = -0.25
    y = bi.bi_rms_norm(x.to(DEV), w.to(DEV), 0.0, out_dtype=bi.BI_F32)
    xi = synth.randint((8, 777), -100, 100, seed=7, dtype=torch.bfloat16)
    m = bi.bi_mean_rows(xi.to(DEV))
    c = bi.bi_log_softmax_rows(torch.full((2, 1024), -7.5, device=DEV))
    _sync()
    assert torch.equal(y.cpu(), torch.sign(x.float()) * w.float())
    exact = torch.tensor(oracle.mean_rows(xi), dtype=torch.float32)   # fp32 rounding of the exact mean
    assert torch.equal(m.cpu(), exact)
    assert np.all(np.abs(to64(c) + math.log(1024.0)) <= 2 ** -20)


def test_llm_shapes_sampled():
    # The bench's shapes: RMSNorm and mean over X [8192, 4096] bf16, log-softmax
    # over the addmm output [8192, 14336] bf16; sampled rows against the oracle.
    x = synth.randn((8192, 4096), seed=8, dtype=torch.bfloat16)
    w = synth.randn((4096,), seed=9, dtype=torch.bfloat16)
    lg = synth.randn((8192, 14336), seed=10, dtype=torch.bfloat16, scale=3.0)
    xd, wd, lgd = x.to(DEV), w.to(DEV), lg.to(DEV)
    y = bi.bi_rms_norm(xd, wd, 1e-6, out_dtype=bi.BI_F32)
    m = bi.bi_mean_rows(xd)
    ls = bi.bi_log_softmax_rows(lgd, out_dtype=bi.BI_F32)
    _sync()
    rows = [0, 1, 4095, 8191]
    assert_parity(to64(y[rows]), oracle.rms_norm(x[rows], w, 1e-6), "rms_norm 8192x4096")
    assert_parity(to64(m[rows])[:, None], oracle.mean_rows(x[rows])[:, None], "mean 8192x4096")
    assert_parity(to64(ls[rows]), oracle.log_softmax_rows(lg[rows]), "log_softmax 8192x14336")


@pytest.mark.parametrize("rows,cols", [(50001, 256), (9001, 4096), (3, 1000)])
def test_rms_norm_rows_beyond_one_pass(rows, cols):
    # More rows than one pass of the resident grid: each wave normalises
    # several rows in turn.  Sampled rows equal the same row normalised alone,
    # bit for bit, and match the oracle.
    x = synth.randn((rows, cols), seed=rows + cols, dtype=torch.bfloat16).to(DEV)
    w = synth.randn((cols,), seed=7, dtype=torch.bfloat16).to(DEV)
    y = bi.bi_rms_norm(x, w, 1e-6, out_dtype=bi.BI_F32)
    gen = np.random.default_rng(rows)
    pick = sorted({0, rows - 1, *gen.integers(0, rows, 30).tolist()})
    alone = [bi.bi_rms_norm(x[r:r + 1], w, 1e-6, out_dtype=bi.BI_F32) for r in pick]
    _sync()
    for r, a in zip(pick, alone):
        assert bitwise_equal(y[r:r + 1], a), f"row {r} of {rows} differs from the row alone"
    idx = torch.tensor(pick)
    assert_parity(to64(y.cpu()[idx]), oracle.rms_norm(x.cpu()[idx], w.cpu(), 1e-6), f"rms_norm {rows}x{cols} sampled")

"""Comparison helpers for the GPU parity tests.

Tolerance (binary32 outputs against the fp64 oracle, on the same inputs):
relative L2 error <= 1e-5 over the checked tensor and, for every output row
(the outputs that share one reduction input), max |got - ref| <= 1e-4 *
||ref row||_2.  A bfloat16 output is checked as a rounding decision: every
element must equal RNE(x) for some x within that same per-row bound of the
oracle value, i.e. lie between RNE(ref - band) and RNE(ref + band).
"""
import json
import os

import numpy as np
import torch

import oracle

REL_L2 = 1e-5
ROW_MAXABS = 1e-4


def to64(t):
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 else \
        t.detach().cpu().double().numpy()


def rel_l2(got, ref):
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / n) if n > 0 else float(np.linalg.norm(got))


def assert_parity(got, ref, what="", rel=REL_L2, row=ROW_MAXABS):
    """got, ref: float64 arrays whose LAST axis is the output row."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    e = rel_l2(got, ref)
    assert e <= rel, f"{what}: relative L2 {e:.3e} > {rel:.0e}"
    g2 = got.reshape(-1, got.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    err = np.abs(g2 - r2).max(1)
    bound = row * np.linalg.norm(r2, axis=1)
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (f"{what}: {bad.size} rows exceed max-abs {row:.0e}*||row||; worst row "
                           f"{bad[0]} err {err[bad[0]]:.3e} bound {bound[bad[0]]:.3e}")
    return e


def assert_bf16_rounding(got_bf16, ref, what="", row=ROW_MAXABS):
    """got_bf16: bfloat16 tensor; ref: float64 oracle array, last axis = row."""
    g = to64(got_bf16).reshape(-1, ref.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    band = row * np.linalg.norm(r, axis=1, keepdims=True)
    lo = oracle.bf16_rne_array(r - band)
    hi = oracle.bf16_rne_array(r + band)
    bad = np.nonzero((g < lo) | (g > hi))
    assert bad[0].size == 0, (f"{what}: {bad[0].size} bf16 outputs are not a rounding of a value "
                              f"within tolerance; first at {bad[0][0]},{bad[1][0]}: got "
                              f"{g[bad][0]} ref {r[bad][0]}")


def assert_bf16_is_rne_of(got_bf16, got_f32, what=""):
    """The bfloat16 output is bit for bit the RNE rounding of the binary32 output."""
    ref = got_f32.to(torch.bfloat16)
    assert torch.equal(got_bf16.view(torch.int16), ref.view(torch.int16)), \
        f"{what}: bf16 output differs from RNE(fp32 output)"


def bitwise_equal(a, b):
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    iv = {2: torch.int16, 4: torch.int32, 8: torch.int64}[a.element_size()]
    return torch.equal(a.view(iv), b.view(iv))


def assert_within_dot_bound(got, ref, mag, K, what=""):
    """Forward error bound of a binary32 sum of K products (exact products, as
    bf16 x bf16 is exact in binary32): |got - ref| <= gamma_K * sum_k |a_k b_k|,
    gamma_K = K u / (1 - K u), u = 2^-24."""
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    err = np.abs(np.asarray(got) - np.asarray(ref))
    bound = gamma * np.asarray(mag)
    assert np.all(err <= bound), f"{what}: error {err.max():.3e} exceeds gamma_K bound"


def comparison_record(got, ref, what=""):
    """The comparison figures of the VLA page's tracer ("Batch-Invariant
    VLAs", section "Profiling batch-invariance"): max_abs_diff, mean_abs_diff,
    rmse, relative_l2_mean / relative_l2_max (relative L2 per sample, the
    first axis, then the mean and maximum over samples) and output_abs_max.
    got, ref: arrays of the same shape, first axis = sample.  When the
    environment names a file in BI_COMPARISON_RECORD the record is appended
    to it as one JSON line."""
    g = np.asarray(got, dtype=np.float64).reshape(len(got), -1)
    r = np.asarray(ref, dtype=np.float64).reshape(len(ref), -1)
    d = g - r
    nr = np.linalg.norm(r, axis=1)
    rel = np.linalg.norm(d, axis=1) / np.where(nr > 0, nr, 1.0)
    rec = {"what": what, "samples": int(g.shape[0]),
           "max_abs_diff": float(np.abs(d).max()) if d.size else 0.0,
           "mean_abs_diff": float(np.abs(d).mean()) if d.size else 0.0,
           "rmse": float(np.sqrt((d * d).mean())) if d.size else 0.0,
           "relative_l2_mean": float(rel.mean()) if rel.size else 0.0,
           "relative_l2_max": float(rel.max()) if rel.size else 0.0,
           "output_abs_max": float(np.abs(g).max()) if g.size else 0.0}
    path = os.environ.get("BI_COMPARISON_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
    return rec

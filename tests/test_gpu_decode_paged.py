"""GPU parity and invariance of bi_decode_attn_paged (through the C ABI).

Requests of their own lengths read K and V through a block table from a paged
cache [num_pages, H, P, D].  Each request must match the unsplit fp64 oracle
(reading the same pages) and give, bit for bit, what bi_decode_attn gives for
that request alone with its K and V stored contiguously (S = its length), for
page sizes on both addressing paths (P below and at least the tokens of one
wave-wide load), D = 64 and 128, and lengths around the page and the 2048-token
chunk boundaries.  A request's bits do not depend on the other requests, the
table width, max_seq_len or where its pages sit.  Edge cases: length 0 gives
NaN; a length above max_seq_len is clamped to it; a page id outside the cache
reads page 0.  The bench shape (256 requests, 32 heads, D = 64, P = 16,
lengths up to 8192) is checked on sampled requests.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_bf16_rounding, assert_parity, bitwise_equal, to64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
DEV = "cuda"
LENS = [1, 3, 15, 16, 17, 100, 2047, 2048, 2049, 4100]


def _paged(q, kc, vc, bt, sl, max_seq, scale, **kw):
    return bi.bi_decode_attn_paged(q, kc, vc, bt, sl, max_seq, scale, **kw)


@pytest.mark.parametrize("D,P", [(64, 16), (64, 8), (64, 4), (64, 1), (64, 256), (64, 4096),
                                 (128, 16), (128, 4), (128, 2), (128, 1)])
def test_paged_parity_and_equal_to_contiguous(D, P):
    H = 3
    scale = float(np.float32(1.0 / np.sqrt(D)))
    q, kc, vc, bt, sl, ks, vs = synth.paged_decode_inputs(LENS, H=H, D=D, P=P, seed=D + P)
    max_seq = max(LENS)
    dq, dk, dv, dbt, dsl = (t.to(DEV) for t in (q, kc, vc, bt, sl))
    o32 = _paged(dq, dk, dv, dbt, dsl, max_seq, scale, out_dtype=bi.BI_F32)
    o16 = _paged(dq, dk, dv, dbt, dsl, max_seq, scale, out_dtype=bi.BI_BF16)
    alone = [bi.bi_decode_attn(dq[b:b + 1].contiguous(), ks[b][None].contiguous().to(DEV),
                               vs[b][None].contiguous().to(DEV), scale) for b in range(len(LENS))]
    torch.cuda.synchronize()
    ref = oracle.decode_paged(q, kc, vc, bt, sl, scale)
    assert_parity(to64(o32), ref, f"paged decode D={D} P={P}")
    assert_bf16_rounding(o16, ref, f"paged decode bf16 D={D} P={P}")
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))
    for b, S in enumerate(LENS):
        assert bitwise_equal(o32[b:b + 1], alone[b]), f"request {b} (len {S}) differs from contiguous"


def test_paged_request_invariant_to_batch_and_placement():
    D, P, H = 64, 16, 4
    scale = 0.125
    # Request of length 3000 alone, then first of a batch with longer requests
    # (wider table, larger max_seq_len), then with its pages moved elsewhere.
    q, kc, vc, bt, sl, ks, vs = synth.paged_decode_inputs([3000, 9000, 1, 6000, 2048], H=H, D=D, P=P, seed=5)
    dq, dk, dv, dbt, dsl = (t.to(DEV) for t in (q, kc, vc, bt, sl))
    full = _paged(dq, dk, dv, dbt, dsl, 9000, scale)
    alone = _paged(dq[:1].contiguous(), dk, dv, dbt[:1, :188].contiguous(), dsl[:1].contiguous(), 3000, scale)
    wide = torch.full((5, 1300), -1, dtype=torch.int32)
    wide[:, :bt.shape[1]] = bt
    loose = _paged(dq, dk, dv, wide.to(DEV), dsl, 20000, scale)   # wider table, larger max_seq_len
    n = kc.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(9))
    kc2, vc2 = torch.empty_like(kc), torch.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0).long()].to(torch.int32), bt)
    moved = _paged(dq, kc2.to(DEV), vc2.to(DEV), bt2.to(DEV), dsl, 9000, scale)
    torch.cuda.synchronize()
    assert bitwise_equal(full[:1], alone), "request 0 depends on the batch"
    assert bitwise_equal(full, loose), "table width or max_seq_len changes the bits"
    assert bitwise_equal(full, moved), "page placement changes the bits"


def test_paged_edge_cases():
    D, P, H = 64, 16, 2
    q, kc, vc, bt, sl, ks, vs = synth.paged_decode_inputs([0, 40, 700], H=H, D=D, P=P, seed=6)
    dq, dk, dv, dbt = (t.to(DEV) for t in (q, kc, vc, bt))
    o = _paged(dq, dk, dv, dbt, sl.to(DEV), 700, 0.125)
    # A length above max_seq_len (here 900 > 700) is clamped to max_seq_len.
    over = _paged(dq, dk, dv, dbt, torch.tensor([0, 40, 900], dtype=torch.int32, device=DEV), 700, 0.125)
    # Page ids outside [0, num_pages) read page 0.
    bad = bt.clone()
    bad[1, 1] = -5
    bad[2, 3] = kc.shape[0] + 100
    zero = bt.clone()
    zero[1, 1] = 0
    zero[2, 3] = 0
    ob = _paged(dq, dk, dv, bad.to(DEV), sl.to(DEV), 700, 0.125)
    oz = _paged(dq, dk, dv, zero.to(DEV), sl.to(DEV), 700, 0.125)
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(o[0])), "length 0 must give NaN"
    assert torch.all(torch.isfinite(o[1:]))
    assert bitwise_equal(o[1:], over[1:]), "length above max_seq_len not clamped"
    assert bitwise_equal(ob, oz), "out-of-range page id must read page 0"


def test_paged_bench_shape_sampled():
    B, H, D, P = 256, 32, 64, 16
    g = torch.Generator().manual_seed(11)
    lens = torch.randint(1, 8193, (B,), generator=g)
    lens[0], lens[1] = 8192, 1
    lens = lens.tolist()
    q, kc, vc, bt, sl, _, _ = synth.paged_decode_inputs(lens, H=H, D=D, P=P, seed=12, device=DEV,
                                                        with_seq=False)
    o = _paged(q, kc, vc, bt, sl, 8192, 0.125)
    torch.cuda.synchronize()
    for b in (0, 1, 77, 255):
        k, v = synth.request_kv(kc, vc, bt, sl, b)
        alone = bi.bi_decode_attn(q[b:b + 1].contiguous(), k, v, 0.125)
        torch.cuda.synchronize()
        assert bitwise_equal(o[b:b + 1], alone), f"request {b} (len {lens[b]}) differs from contiguous"
        ref = oracle.decode(q[b:b + 1].cpu(), k.cpu(), v.cpu(), 0.125)
        assert_parity(to64(o[b:b + 1]), ref, f"paged bench shape request {b}")

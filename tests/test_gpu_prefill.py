"""GPU parity and invariance of bi_prefill_attn_paged (through the C ABI).

Causal prefill over a paged cache, KV split at 4096 tokens.  Parity with the
unsplit fp64 oracle on requests whose positions cross the 4096-token split
(prefix-cache hits, ragged chunk lengths, a one-token chunk); bit-for-bit
invariance to the way a prompt is cut into prefill chunks, to the other
requests of the batch and the grid bounds (max_q, max_kv_len), and to the
page size and page placement; sampled rows of an 8192-token prompt.
"""
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
SCALE = float(np.float32(1.0 / np.sqrt(128.0)))


def _dev(*ts):
    return [t.to(DEV) for t in ts]


def _run(q, cu, p0, kc, vc, bt, max_q=None, max_kv=None, **kw):
    n = (cu[1:] - cu[:-1]).max().item()
    kv = (p0 + (cu[1:] - cu[:-1])).max().item()
    return bi.bi_prefill_attn_paged(q, cu, p0, max_q or n, kc, vc, bt, max_kv or kv, SCALE, **kw)


@pytest.mark.parametrize("case", ["fresh", "prefix_hits", "cross_split"])
def test_prefill_parity(case):
    prefix, n = {"fresh": ([0, 0], [300, 1]),
                 "prefix_hits": ([37, 1000, 255], [100, 17, 1]),
                 "cross_split": ([4000, 3900, 8000], [200, 300, 250])}[case]
    q, cu, p0, kc, vc, bt = synth.paged_prefill_inputs(prefix, n, H=2, D=128, P=16, seed=len(case))
    dq, dcu, dp0, dkc, dvc, dbt = _dev(q, cu, p0, kc, vc, bt)
    o32 = _run(dq, dcu, dp0, dkc, dvc, dbt)
    o16 = _run(dq, dcu, dp0, dkc, dvc, dbt, out_dtype=bi.BI_BF16)
    torch.cuda.synchronize()
    ref = oracle.prefill_paged(q, cu, p0, kc, vc, bt, SCALE)
    assert_parity(to64(o32), ref, f"prefill {case}")
    assert_bf16_is_rne_of(o16, o32, f"prefill {case} bf16")


def test_chunked_prefill_same_bits():
    # One 5000-token prompt: a single call, then three prefill chunks that
    # each see the earlier tokens as cached prefix.
    q, cu, p0, kc, vc, bt = synth.paged_prefill_inputs([0], [5000], H=2, D=128, P=16, seed=7)
    dq, dkc, dvc, dbt = _dev(q, kc, vc, bt)
    whole = _run(dq, cu.to(DEV), p0.to(DEV), dkc, dvc, dbt)
    parts = []
    for a, e in ((0, 1000), (1000, 4100), (4100, 4101), (4101, 5000)):
        cu_c = torch.tensor([0, e - a], dtype=torch.int32, device=DEV)
        p0_c = torch.tensor([a], dtype=torch.int32, device=DEV)
        parts.append(_run(dq[a:e].contiguous(), cu_c, p0_c, dkc, dvc, dbt))
    torch.cuda.synchronize()
    assert bitwise_equal(whole, torch.cat(parts)), "chunked prefill changes the bits"


def test_prefill_batch_and_bounds_invariance():
    prefix, n = [500, 0, 4090, 7], [260, 33, 600, 1]
    q, cu, p0, kc, vc, bt = synth.paged_prefill_inputs(prefix, n, H=3, D=128, P=16, seed=8)
    dq, dcu, dp0, dkc, dvc, dbt = _dev(q, cu, p0, kc, vc, bt)
    full = _run(dq, dcu, dp0, dkc, dvc, dbt)
    loose = _run(dq, dcu, dp0, dkc, dvc, torch.cat([dbt, torch.full_like(dbt, -1)], 1),
                 max_q=2000, max_kv=9000)
    alone = []
    for b in range(4):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        cu_b = torch.tensor([0, r1 - r0], dtype=torch.int32, device=DEV)
        alone.append(_run(dq[r0:r1].contiguous(), cu_b, dp0[b:b + 1].contiguous(), dkc, dvc,
                          dbt[b:b + 1].contiguous()))
    torch.cuda.synchronize()
    assert bitwise_equal(full, loose), "grid bounds change the bits"
    assert bitwise_equal(full, torch.cat(alone)), "a request's bits depend on the batch"


def test_prefill_page_size_and_placement_invariance():
    # The same K and V stored with page sizes 1, 4, 16, 64 and a shuffled placement.
    q, cu, p0, kc, vc, bt = synth.paged_prefill_inputs([100, 0], [300, 129], H=2, D=128, P=16, seed=9)
    outs = []
    for P in (1, 4, 16, 64):
        B = 2
        kv = [400, 129]
        ks, vs, tabs, pages = [], [], [], 0
        for b in range(B):
            k, v = synth.request_kv(kc, vc, bt, torch.tensor(kv, dtype=torch.int32), b)
            npg = (kv[b] + P - 1) // P
            pad = npg * P - kv[b]
            k = torch.cat([k[0], torch.zeros(2, pad, 128, dtype=k.dtype)], 1)
            v = torch.cat([v[0], torch.zeros(2, pad, 128, dtype=v.dtype)], 1)
            ks.append(k.view(2, npg, P, 128).permute(1, 0, 2, 3))
            vs.append(v.view(2, npg, P, 128).permute(1, 0, 2, 3))
            tabs.append(list(range(pages, pages + npg)))
            pages += npg
        perm = torch.randperm(pages, generator=torch.Generator().manual_seed(P))
        kc2 = torch.empty(pages, 2, P, 128, dtype=kc.dtype)
        vc2 = torch.empty_like(kc2)
        kc2[perm] = torch.cat(ks)
        vc2[perm] = torch.cat(vs)
        mp = max(len(t) for t in tabs)
        bt2 = torch.full((B, mp), -1, dtype=torch.int32)
        for b in range(B):
            bt2[b, :len(tabs[b])] = perm[torch.tensor(tabs[b])].to(torch.int32)
        outs.append(_run(*_dev(q, cu, p0, kc2, vc2, bt2)))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert bitwise_equal(outs[0], o), "page size or placement changes the bits"


def test_prefill_long_prompt_sampled():
    # One 8192-token prompt, 8 heads: rows around the 4096 split and the ends.
    H = 8
    q, cu, p0, kc, vc, bt = synth.paged_prefill_inputs([0], [8192], H=H, D=128, P=16, seed=10, device=DEV)
    o = _run(q, cu, p0, kc, vc, bt)
    torch.cuda.synchronize()
    rows = [0, 1, 255, 256, 4095, 4096, 4097, 6000, 8191]
    qs = q[rows].cpu()
    cu_s = torch.arange(len(rows) + 1, dtype=torch.int32)
    p0_s = torch.tensor(rows, dtype=torch.int32)
    bt_s = bt.cpu().expand(len(rows), -1).contiguous()
    ref = oracle.prefill_paged(qs, cu_s, p0_s, kc.cpu(), vc.cpu(), bt_s, SCALE)
    assert_parity(to64(o[rows]), ref, "prefill 8192 sampled rows")


def _repage(kc, vc, bt, lens, P, seed):
    """The same tokens of each request in pages of P tokens (a seeded permutation of pages)."""
    P0, H, D = kc.shape[2], kc.shape[1], kc.shape[3]
    npg = [(n + P - 1) // P for n in lens]
    num_pages = sum(npg) + 3
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(num_pages, generator=g)
    kc2 = torch.zeros((num_pages, H, P, D), dtype=kc.dtype)
    vc2 = torch.zeros_like(kc2)
    bt2 = torch.full((len(lens), max(npg)), -1, dtype=torch.int32)
    used = 0
    for b, n in enumerate(lens):
        t = torch.arange(n)
        src_page, src_slot = bt[b, t // P0].long(), t % P0
        pages = perm[used:used + npg[b]]
        used += npg[b]
        bt2[b, :npg[b]] = pages.to(torch.int32)
        dst_page, dst_slot = pages[t // P], t % P
        for c2, c in ((kc2, kc), (vc2, vc)):
            c2[dst_page, :, dst_slot, :] = c[src_page, :, src_slot, :]
    return kc2, vc2, bt2


@pytest.mark.parametrize("P", [1, 4, 8, 32, 64, 128])
def test_page_size_does_not_change_the_bits(P):
    # Pages only place the tokens: every page size gives the bits of 16-token
    # pages (the copies take a uniform page per 16 keys for pages of 16 or
    # more tokens and per-lane pages below, and chunks start inside pages of
    # 128); prefix hits, a chunk crossing 4096 and ragged lengths.
    prefix, n = [37, 1000, 4000], [100, 17, 300]
    lens = [a + b for a, b in zip(prefix, n)]
    q, cu, p0, kc, vc, bt = synth.paged_prefill_inputs(prefix, n, H=2, D=128, P=16, seed=11)
    ref = _run(*_dev(q, cu, p0, kc, vc, bt))
    kc2, vc2, bt2 = _repage(kc, vc, bt, lens, P, seed=100 + P)
    got = _run(*_dev(q, cu, p0, kc2, vc2, bt2))
    torch.cuda.synchronize()
    assert bitwise_equal(got, ref), f"pages of {P} tokens changed the bits"

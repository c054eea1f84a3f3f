"""Pins of the oracle's paged decode (CPU only).

The paged oracle reads K and V through the block table; it must give exactly
the unsplit decode oracle's result on the same values stored contiguously
(gathered here with torch indexing, independently of the oracle), for every
request at its own length; the physical page assignment must not matter; and
a request of one token returns that token's V row exactly.
"""
import numpy as np
import torch

import oracle
import synth


def test_paged_equals_contiguous_per_request():
    lens = [1, 15, 16, 17, 300, 2048, 2049, 4100]
    q, kc, vc, bt, sl, ks, vs = synth.paged_decode_inputs(lens, H=3, D=64, P=16, seed=1)
    got = oracle.decode_paged(q, kc, vc, bt, sl, 0.125)
    for b, S in enumerate(lens):
        ref = oracle.decode(q[b:b + 1], ks[b][None], vs[b][None], 0.125)
        assert np.array_equal(got[b:b + 1], ref), f"request {b} (S={S})"


def test_paged_page_assignment_does_not_matter():
    lens = [700, 33]
    a = synth.paged_decode_inputs(lens, H=2, D=64, P=32, seed=2)
    q, kc, vc, bt, sl = a[:5]
    # Move every page to a new physical slot (reverse order) and rewrite the table.
    n = kc.shape[0]
    perm = torch.arange(n - 1, -1, -1)
    kc2, vc2 = torch.empty_like(kc), torch.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0).long()].to(torch.int32), bt)
    assert np.array_equal(oracle.decode_paged(q, kc, vc, bt, sl, 0.125),
                          oracle.decode_paged(q, kc2, vc2, bt2, sl, 0.125))


def test_single_token_request_returns_its_value_row():
    q, kc, vc, bt, sl, ks, vs = synth.paged_decode_inputs([1, 1], H=2, D=64, P=16, seed=3)
    got = oracle.decode_paged(q, kc, vc, bt, sl, 0.125)
    for b in range(2):
        assert np.array_equal(got[b], vs[b][:, 0].double().numpy())

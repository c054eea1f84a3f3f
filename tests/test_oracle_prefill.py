"""Pins of the oracle's causal prefill over a paged cache (CPU only).

A query at position pos attends to keys 0 .. pos of its own request.  Pinned
by: a single query at the end of a request equals the paged decode oracle (at
the request's length) bit for bit; torch float64 causal attention on K and V
gathered with torch indexing; cutting a prompt into prefill chunks (each chunk's
queries with the right starting position) gives the same bits as one call;
V = 1 gives 1 exactly; q = 0 averages V over keys 0 .. pos exactly (small
integers), which fails for an off-by-one causal bound.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle
import synth


def _gather(kc, vc, bt, b, S):
    P = kc.shape[2]
    pages = bt[b, :(S + P - 1) // P].long()
    H, D = kc.shape[1], kc.shape[3]
    k = kc[pages].permute(1, 0, 2, 3).reshape(H, -1, D)[:, :S]
    v = vc[pages].permute(1, 0, 2, 3).reshape(H, -1, D)[:, :S]
    return k, v


def test_last_query_equals_paged_decode():
    prefix, n = [0, 5, 40, 2000], [7, 1, 9, 3]
    q, cu, p0, kc, vc, bt = synth.paged_prefill_inputs(prefix, n, H=2, D=64, P=16, seed=1)
    out = oracle.prefill_paged(q, cu, p0, kc, vc, bt, 0.125)
    last = cu[1:].long() - 1
    lens = torch.tensor([a + m for a, m in zip(prefix, n)], dtype=torch.int32)
    dec = oracle.decode_paged(q[last], kc, vc, bt, lens, 0.125)
    assert np.array_equal(out[last.numpy()], dec)


def test_matches_torch_float64_causal_attention():
    prefix, n = [0, 33, 100], [20, 16, 5]
    q, cu, p0, kc, vc, bt = synth.paged_prefill_inputs(prefix, n, H=3, D=32, P=8, seed=2)
    out = oracle.prefill_paged(q, cu, p0, kc, vc, bt, 0.2)
    for b in range(3):
        S = prefix[b] + n[b]
        k, v = _gather(kc, vc, bt, b, S)
        qb = q[cu[b]:cu[b + 1]].double().permute(1, 0, 2)          # [H, n, D]
        s = 0.2 * torch.matmul(qb, k.double().transpose(1, 2))       # [H, n, S]
        pos = prefix[b] + torch.arange(n[b])
        s = s.masked_fill(torch.arange(S)[None, None, :] > pos[None, :, None], float("-inf"))
        ref = torch.matmul(torch.softmax(s, -1), v.double()).permute(1, 0, 2)
        got = out[int(cu[b]):int(cu[b + 1])]
        assert np.max(np.abs(got - ref.numpy())) <= 1e-12 * np.abs(ref.numpy()).max()


def test_chunked_prefill_gives_the_same_bits():
    # One request with a 300-token prompt: once, then as chunks 0..99, 100..249, 250..299.
    q, cu, p0, kc, vc, bt = synth.paged_prefill_inputs([0], [300], H=2, D=64, P=16, seed=3)
    whole = oracle.prefill_paged(q, cu, p0, kc, vc, bt, 0.125)
    parts = []
    for a, e in ((0, 100), (100, 250), (250, 300)):
        parts.append(oracle.prefill_paged(q[a:e], [0, e - a], [a], kc, vc, bt, 0.125))
    assert np.array_equal(whole, np.concatenate(parts))


def test_closed_forms_and_causal_bound():
    q, cu, p0, kc, vc, bt = synth.paged_prefill_inputs([3], [12], H=2, D=16, P=4, seed=4)
    ones = torch.ones_like(vc)
    assert np.all(oracle.prefill_paged(q, cu, p0, kc, ones, bt, 0.3) == 1.0)
    vi = synth.randint(tuple(vc.shape), -9, 9, seed=5, dtype=torch.bfloat16)
    out = oracle.prefill_paged(torch.zeros_like(q), cu, p0, kc, vi, bt, 0.3)
    _, v = _gather(kc, vi, bt, 0, 15)
    for j in range(12):
        pos = 3 + j
        for h in range(2):
            exact = [float(Fraction(int(x)) / (pos + 1)) for x in v[h, :pos + 1].double().sum(0)]
            assert out[j, h].tolist() == exact

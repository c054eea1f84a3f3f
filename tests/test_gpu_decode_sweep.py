"""Seeded random sweep of the paged decode (through the C ABI).

Each case draws the request count, per-request lengths (short ones, ones
around the page and 2048-token chunk boundaries, long ones), heads, head
dimension and page size from its seed.  Every request matches the unsplit
fp64 oracle and equals, bit for bit, bi_decode_attn on that request alone
with its K and V stored contiguously ("Unmasking the True Culprit ...",
section "Why This Achieves Batch Invariance": the split depends on the
request's own length only; the deterministic-inference handbook, section
"与 batch 无关：固定切分": fixed-size chunks).
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
CASES = 20


def _case(seed):
    rng = np.random.default_rng(11000 + seed)
    B = int(rng.integers(1, 7))
    lens = []
    for _ in range(B):
        kind = int(rng.integers(0, 3))
        if kind == 0:
            lens.append(int(rng.integers(1, 64)))
        elif kind == 1:
            lens.append(int(rng.choice([2047, 2048, 2049, 4095, 4096, 4097])) + int(rng.integers(-2, 3)))
        else:
            lens.append(int(rng.integers(64, 9000)))
    return dict(lens=lens, H=int(rng.choice([1, 2, 3, 5])), D=int(rng.choice([64, 128])),
                P=int(rng.choice([1, 2, 4, 8, 16, 32, 64, 256])))


@pytest.mark.parametrize("seed", range(CASES))
def test_random_paged_decode(seed):
    c = _case(seed)
    name = f"seed {seed}: {c}"
    print(name, flush=True)
    lens, H, D, P = c["lens"], c["H"], c["D"], c["P"]
    scale = float(np.float32(1.0 / np.sqrt(D)))
    q, kc, vc, bt, sl, ks, vs = synth.paged_decode_inputs(lens, H=H, D=D, P=P, seed=seed)
    dq, dk, dv, dbt, dsl = (t.to(DEV) for t in (q, kc, vc, bt, sl))
    out = bi.bi_decode_attn_paged(dq, dk, dv, dbt, dsl, max(lens), scale, out_dtype=bi.BI_F32)
    alone = [bi.bi_decode_attn(dq[b:b + 1].contiguous(), ks[b][None].contiguous().to(DEV),
                               vs[b][None].contiguous().to(DEV), scale) for b in range(len(lens))]
    torch.cuda.synchronize()
    assert_parity(to64(out), oracle.decode_paged(q, kc, vc, bt, sl, scale), name)
    for b in range(len(lens)):
        assert bitwise_equal(out[b:b + 1], alone[b]), f"{name}: request {b} differs from it alone"

"""GPU checks of the benchmark variants (libbi_bench.so).

* The invariant GEMM gives the same bits on any persistent grid (1, 7, 256
  workgroups): which workgroup runs a tile does not enter the arithmetic.
* Negative controls: a batch-size-tuned split-K GEMM and a load-based split-KV
  decode are correct (they match the oracle) but NOT batch invariant, and
  reproduce on the GPU the patterns the deterministic-inference handbook
  prints for its CPU experiments (section "根源：浮点加法的顺序"): split-K by M
  gives row 0 equal to "alone" for M = 8, 63 and different for M = 64, 200;
  splits by load (132 units) give request 0 equal to batch 1 only at B = 1.
  This shows the invariance tests can see a changed reduction order.
* The addmm with dispatch-attached events (the benchmark's timing of its
  headline kernel) gives bi_addmm's bits.
* The wave-wide reduction shared by the softmax, the row operations and the
  attention probabilities adds in the xor-butterfly order, bit for bit.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_parity, bitwise_equal, to64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
    from invariant_persistent_bf16_amd import bi_bench
DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("b_layout", ["n_contig", "k_contig"])
def test_gemm_grid_independent(b_layout):
    M, N, K = 600, 776, 320
    A = synth.randn((M, K), seed=1, dtype=torch.bfloat16).to(DEV)
    B = synth.randn((K, N), seed=2, dtype=torch.bfloat16).to(DEV)
    if b_layout == "k_contig":
        B = B.t().contiguous().t()
    bias = synth.randn((N,), seed=3, dtype=torch.bfloat16).to(DEV)
    ref = bi.bi_addmm(bias, A, B, out_dtype=bi.BI_F32)
    outs = [bi_bench.gemm_grid(A, B, g, bias=bias, out_dtype=bi.BI_F32) for g in (1, 7, 256, 1000)]
    torch.cuda.synchronize()
    for g, o in zip((1, 7, 256, 1000), outs):
        assert bitwise_equal(o, ref), f"grid {g} changed the result"


def test_fp32_gemm_grid_independent():
    A = synth.randn((130, 300), seed=4).to(DEV)
    B = synth.randn((300, 200), seed=5).to(DEV)
    ref = bi.bi_mm(A, B)
    outs = [bi_bench.gemm_grid(A, B, g) for g in (1, 3, 64)]
    torch.cuda.synchronize()
    assert all(bitwise_equal(o, ref) for o in outs)


def test_splitk_handbook_rule_pattern_on_gpu():
    g = json.load(open(os.path.join(GOLDEN, "handbook_splitk_gemm.json")))
    W, bias, x0 = synth.addmm_shared(N=2048)
    Wd, bd = W.to(DEV), bias.to(DEV)
    alone_X = x0.to(DEV)
    alone = bi_bench.addmm_splitk(bd, alone_X, Wd, bi_bench.splitk_policy(1, 2048, 4096, rule=1),
                                  out_dtype=bi.BI_F32)
    got = []
    for M in g["batches"]:
        X = synth.addmm_batch(x0, M, device=DEV)
        s = bi_bench.splitk_policy(M, 2048, 4096, rule=1)
        C = bi_bench.addmm_splitk(bd, X, Wd, s, out_dtype=bi.BI_F32)
        torch.cuda.synchronize()
        got.append(bitwise_equal(C[0], alone[0]))
        assert_parity(to64(C[:4]), oracle.mm(X[:4].cpu(), W, bias), f"split-K M={M}")
    assert got == g["row0_equals_alone_by_batch"]
    # The invariant kernel on the same inputs: always equal.
    inv_alone = bi.bi_addmm(bd, alone_X, Wd, out_dtype=bi.BI_F32)
    for M in g["batches"]:
        X = synth.addmm_batch(x0, M, device=DEV)
        C = bi.bi_addmm(bd, X, Wd, out_dtype=bi.BI_F32)
        torch.cuda.synchronize()
        assert bitwise_equal(C[0], inv_alone[0])


def test_splitk_fill_policy_breaks_invariance_at_full_shape():
    W, bias, x0 = synth.addmm_shared()
    Wd, bd = W.to(DEV), bias.to(DEV)
    s1 = bi_bench.splitk_policy(1, 14336, 4096, rule=0)
    s8k = bi_bench.splitk_policy(8192, 14336, 4096, rule=0)
    assert s1 > 1 and s8k == 1
    c1 = bi_bench.addmm_splitk(bd, x0.to(DEV), Wd, s1, out_dtype=bi.BI_F32)
    X = synth.addmm_batch(x0, 8192, device=DEV)
    c8k = bi_bench.addmm_splitk(bd, X, Wd, s8k, out_dtype=bi.BI_F32)
    inv = bi.bi_addmm(bd, X, Wd, out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    assert not bitwise_equal(c1[0], c8k[0]), "the negative control should change row 0"
    assert bitwise_equal(c8k, inv), "one split is the invariant kernel"
    assert_parity(to64(c1), oracle.mm(x0, W, bias), "split-K M=1")


def test_decode_by_load_pattern_on_gpu():
    g = json.load(open(os.path.join(GOLDEN, "handbook_decode_splits.json")))
    q, k, v = synth.decode_shared(H=4)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    splits = [bi_bench.decode_splits_policy(b, 132) for b in g["batches"]]
    assert splits == g["splits_by_load"]
    outs = [bi_bench.decode_attn_splits(qd, kd, vd, 0.125, s) for s in splits]
    fixed = bi.bi_decode_attn(qd, kd, vd, 0.125)
    torch.cuda.synchronize()
    got = [bitwise_equal(o, outs[0]) for o in outs]
    assert got == g["equal_to_batch1_by_load"]
    ref = oracle.decode(q, k, v, 0.125)
    for s, o in zip(splits, outs):
        assert_parity(to64(o), ref, f"decode {s} splits")
    # Four equal parts of 2048 are the invariant path's chunks: same bits.
    assert bitwise_equal(bi_bench.decode_attn_splits(qd, kd, vd, 0.125, 4), fixed)


def test_read_probe_runs():
    buf = torch.zeros(1 << 24, dtype=torch.uint8, device=DEV)
    sink = torch.empty(65536, dtype=torch.int32, device=DEV)
    bi_bench.read_probe(buf, sink)
    torch.cuda.synchronize()


def test_row_step_read_runs_and_reduces_the_same_data():
    # The same 2 MiB (four tiles) read in 64- and 128-byte row steps:
    # the xor of a workgroup's 256 words covers the same pieces whatever the
    # step, and equals that of the pieces computed on the host.
    gen = torch.Generator().manual_seed(3)
    host = torch.randint(0, 1 << 30, ((1 << 21) // 4,), dtype=torch.int32, generator=gen)
    buf = host.to(DEV)
    sinks = []
    for b in (64, 128):
        sink = torch.zeros(256 * 256, dtype=torch.int32, device=DEV)
        bi_bench.row_step_read(buf, b, sink)
        sinks.append(sink)
    torch.cuda.synchronize()
    words = [np.bitwise_xor.reduce(x.cpu().numpy().reshape(256, 256), axis=1) for x in sinks]
    assert all(np.array_equal(words[0], w) for w in words[1:])
    pieces = host.numpy().reshape(4, -1, 4)            # tile, 16-byte piece, word
    want = np.bitwise_xor.reduce(pieces[:, :, 0] ^ pieces[:, :, 3], axis=1)
    assert np.array_equal(words[0][:4], want)
    with pytest.raises(Exception):
        bi_bench.row_step_read(buf, 96, sinks[0])
    with pytest.raises(Exception):
        bi_bench.row_step_read(buf[:1000], 64, sinks[0])


@pytest.mark.parametrize("M", [1, 200, 2048])
def test_addmm_events_same_bits_and_kernel_time(M):
    # bi_bench_addmm_events is bi_addmm with events attached to the GEMM
    # dispatch: the same bits, and a kernel time no longer than events
    # recorded around the call.
    N, K = 1024, 512
    A = synth.randn((M, K), seed=41, dtype=torch.bfloat16).to(DEV)
    B = synth.randn((K, N), seed=42, dtype=torch.bfloat16, scale=0.05).to(DEV)
    bias = synth.randn((N,), seed=43, dtype=torch.bfloat16).to(DEV)
    ref = bi.bi_addmm(bias, A, B)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    o0, o1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for e in (k0, k1):
        e.record()
    torch.cuda.synchronize()
    o0.record()
    got = bi_bench.addmm_events(bias, A, B, k0, k1)
    o1.record()
    torch.cuda.synchronize()
    assert bitwise_equal(got, ref), f"addmm_events differs from bi_addmm at M={M}"
    t_kernel, t_call = k0.elapsed_time(k1), o0.elapsed_time(o1)
    print(f"M={M}: kernel {t_kernel * 1e3:.1f} us, around the call {t_call * 1e3:.1f} us", flush=True)
    assert 0.0 < t_kernel <= t_call
    with pytest.raises(ValueError):
        bi_bench.addmm_events(bias, A, B, torch.cuda.Event(enable_timing=True), k1)


@pytest.mark.parametrize("B,D", [(1, 64), (2, 128), (5, 64)])
def test_splitkv_decode_correct_and_fixed_chunks_reproduce_the_product(B, D):
    # The load-split decode (parts merged in the same launch) is correct for
    # every split count, deterministic across calls (its counters reset
    # themselves), and with 2048-token parts it is the product's arithmetic:
    # bi_decode_attn's bits.
    H, S = 4, 8192
    q = synth.randn((B, H, D), seed=61, dtype=torch.bfloat16).to(DEV)
    k = synth.randn((B, H, S, D), seed=62, dtype=torch.bfloat16).to(DEV)
    v = synth.randn((B, H, S, D), seed=63, dtype=torch.bfloat16).to(DEV)
    ref = oracle.decode(q.cpu(), k.cpu(), v.cpu(), 0.125)
    prod = bi.bi_decode_attn(q, k, v, 0.125)
    for splits in (4, 8, 16, 32):
        ws = bi_bench.decode_splitkv_workspace(B, H, D, splits, DEV)
        o1 = bi_bench.decode_attn_splitkv(q, k, v, 0.125, splits, ws)
        o2 = bi_bench.decode_attn_splitkv(q, k, v, 0.125, splits, ws)
        torch.cuda.synchronize()
        assert bitwise_equal(o1, o2), f"splits={splits}: two calls differ"
        assert_parity(to64(o1), ref, f"split-KV decode splits={splits}")
        if splits == S // 2048:
            assert bitwise_equal(o1, prod), "2048-token parts differ from bi_decode_attn"
        assert torch.count_nonzero(ws[-(B * H):]) == 0, "counters not reset"
    assert bi_bench.decode_splitkv_policy(1, 32, 8192, 256) == 8      # 32 x 8 parts of 1024 fill 256 CUs
    assert bi_bench.decode_splitkv_policy(16, 32, 8192, 256) == 4     # 2048-token parts already fill them


def test_wave_reduction_order_is_the_xor_butterfly():
    # The cross-lane sum shared by the softmax, the row operations and the
    # attention probabilities: at offsets 32, 16, 8, 4, 2, 1 each lane adds
    # the value of lane l ^ o.  Values spread over many binades so that another
    # order of the same additions rounds differently; the binary32 emulation
    # below follows the butterfly step by step (every lane ends equal).
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(64) * 2.0 ** rng.integers(-20, 20, 64)).astype(np.float32)
    s = x.copy()
    lanes = np.arange(64)
    for o in (32, 16, 8, 4, 2, 1):
        s = (s + s[lanes ^ o]).astype(np.float32)
    got_s, got_m = bi_bench.wave_reduce(torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(got_s.cpu().numpy().view(np.uint32), s.view(np.uint32))
    assert np.all(got_m.cpu().numpy() == x.max())
    # a plain left-to-right sum rounds differently on these values, so the
    # check above does see the order
    seq = np.float32(0.0)
    for v in x:
        seq = np.float32(seq + v)
    assert seq != s[0]

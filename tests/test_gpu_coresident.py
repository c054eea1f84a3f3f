"""Bits of the persistent GEMM when its workgroups share compute units.

* Two of the GEMM's own workgroups per compute unit: the 128x128-tile kernel
  built without its LDS reservation (bi_bench_gemm_shared_cu) on a grid of
  twice the compute units must give bi_bmm's bits.  Before the fix of the
  epilogue's register hazard (an accumulator copied into a register that a
  dead, still-pending LDS read then overwrote) this configuration returned
  zeros in a few tiles per launch.
* Another stream's kernels on the same compute units: bi_bmm / bi_addmm on
  one stream while the row operations, decode and the binary32 GEMM (all
  using LDS) run on a second stream of the same priority.
* Allocation on a side stream: the binding allocates workspaces on the
  stream the kernels run on, so an allocation on torch's current stream
  right after the call cannot take a workspace still in use.

Every result is compared bit for bit with the same call run alone.  The
groups of the persistent GEMM compute each tile inside one workgroup
("Unmasking the True Culprit ...", section "Why This Achieves Batch
Invariance"), so nothing about placement may change a bit.
"""
import pytest
import torch

import synth
from helpers import bitwise_equal

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
    from invariant_persistent_bf16_amd import bi_bench
DEV = "cuda"


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _cases():
    """(name, A [G,M,K], B [G,K,N] view, bias or None, out dtype)."""
    Q = synth.randn((32, 1024, 128), seed=11, dtype=torch.bfloat16, device=DEV)
    Kt = synth.randn((32, 1024, 128), seed=12, dtype=torch.bfloat16, device=DEV)
    P = synth.randn((16, 1024, 1024), seed=13, dtype=torch.bfloat16, scale=0.03, device=DEV)
    V = synth.randn((16, 1024, 128), seed=14, dtype=torch.bfloat16, device=DEV)
    X = synth.randn((1, 1024, 4096), seed=15, dtype=torch.bfloat16, device=DEV)
    W = synth.randn((1, 4096, 4096), seed=16, dtype=torch.bfloat16, scale=0.02, device=DEV)
    bias = synth.randn((4096,), seed=17, dtype=torch.bfloat16, scale=0.02, device=DEV)
    return [("QK^T fp32", Q, Kt.transpose(1, 2), None, bi.BI_F32),
            ("PV fp32", P, V, None, bi.BI_F32),
            ("addmm bf16", X, W, bias, bi.BI_BF16),
            ("addmm W^T fp32", X, W.transpose(1, 2).contiguous().transpose(1, 2), bias, bi.BI_F32)]


def _ref(A, B, bias, od):
    if bias is None:
        return bi.bi_bmm(A, B, out_dtype=od)
    return bi.bi_addmm(bias, A[0], B[0], out_dtype=od).unsqueeze(0)


def test_two_gemm_workgroups_per_compute_unit():
    grid = 2 * _cus()
    for name, A, B, bias, od in _cases():
        print(f"shared-CU GEMM: {name} {tuple(A.shape)} x {tuple(B.shape)} grid {grid}", flush=True)
        ref = _ref(A, B, bias, od)
        outs = [bi_bench.gemm_shared_cu(A, B, grid, bias=bias, out_dtype=od) for _ in range(3)]
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert bitwise_equal(o, ref), f"{name}: run {i} with two workgroups per CU differs"


def test_gemm_beside_another_stream():
    cus = _cus()
    side = torch.cuda.Stream()
    main = torch.cuda.Stream()
    assert side.priority == main.priority == 0
    # side-stream work: row operations with an LDS merge, decode, binary32 GEMM
    xr = synth.randn((4096, 8192), seed=21, dtype=torch.bfloat16, device=DEV)
    wr = synth.randn((8192,), seed=22, dtype=torch.bfloat16, device=DEV)
    q = synth.randn((16, 32, 64), seed=23, dtype=torch.bfloat16, device=DEV)
    kv = synth.randn((16, 32, 4096, 64), seed=24, dtype=torch.bfloat16, device=DEV)
    a32 = synth.randn((1024, 1024), seed=25, device=DEV)
    b32 = synth.randn((1024, 1024), seed=26, device=DEV)
    cases = _cases()
    refs = [_ref(A, B, bias, od) for _, A, B, bias, od in cases]
    side_ref = (bi.bi_rms_norm(xr, wr, 1e-6), bi.bi_decode_attn(q, kv, kv, 0.125), bi.bi_mm(a32, b32))
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"concurrent streams: repetition {rep} on {cus} CUs", flush=True)
        side_out = []
        with torch.cuda.stream(side):
            for _ in range(4):
                side_out.append((bi.bi_rms_norm(xr, wr, 1e-6, stream=side),
                                 bi.bi_decode_attn(q, kv, kv, 0.125, stream=side),
                                 bi.bi_mm(a32, b32, stream=side)))
        with torch.cuda.stream(main):
            outs = []
            for name, A, B, bias, od in cases:
                if bias is None:
                    outs.append(bi.bi_bmm(A, B, out_dtype=od, stream=main))
                else:
                    outs.append(bi.bi_addmm(bias, A[0], B[0], out_dtype=od, stream=main).unsqueeze(0))
                # the same product forced onto the 128x128 tile (most room left
                # on each compute unit for the other stream's waves)
                outs.append(bi_bench.gemm_tile(A, B, 3, bias=bias, out_dtype=od, stream=main))
        torch.cuda.synchronize()
        for i, (name, *_rest) in enumerate(cases):
            assert bitwise_equal(outs[2 * i], refs[i]), f"{name}: differs beside another stream"
            assert bitwise_equal(outs[2 * i + 1], refs[i]), f"{name} (128x128): differs beside another stream"
        for so in side_out:
            for got, ref in zip(so, side_ref):
                assert bitwise_equal(got, ref), "side-stream result differs"


def test_side_stream_workspaces_are_not_reused_early():
    side = torch.cuda.Stream()
    w, cb, x0 = synth.conv_shared()
    x = synth.conv_batch(x0, 32, device=DEV)
    wd, cbd = w.to(DEV), cb.to(DEV)
    q = synth.randn((64, 32, 64), seed=31, dtype=torch.bfloat16, device=DEV)
    kv = synth.randn((64, 32, 8192, 64), seed=32, dtype=torch.bfloat16, device=DEV)
    y_ref = bi.bi_conv2d(x, wd, cbd, stride=(14, 14), out_dtype=bi.BI_F32)
    o_ref = bi.bi_decode_attn(q, kv, kv, 0.125)
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"side-stream workspaces: repetition {rep}", flush=True)
        side.wait_stream(torch.cuda.current_stream())
        y = bi.bi_conv2d(x, wd, cbd, stride=(14, 14), out_dtype=bi.BI_F32, stream=side)
        o = bi.bi_decode_attn(q, kv, kv, 0.125, stream=side)
        # the current stream allocates and overwrites fresh memory at once
        junk = [torch.full((1 << 22,), float(i + 1), device=DEV) for i in range(16)]
        torch.cuda.synchronize()
        del junk
        assert bitwise_equal(y, y_ref), "conv on a side stream differs"
        assert bitwise_equal(o, o_ref), "decode on a side stream differs"

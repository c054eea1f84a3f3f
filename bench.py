#!/usr/bin/env python3
"""Benchmark of the batch-invariant contraction path on one MI355X.

One step runs every operation of the path once, on inputs already resident
in HBM (seeded synthetic data of the pages' workload shapes):
  * addmm   bf16  X [8192, 4096] @ W [4096, 14336] + bias -> bf16   (the large GEMM)
  * conv2d  bf16  SigLIP patch embedding, 32 images 3x224x224 -> [32, 1152, 16, 16]
  * attention bf16, B=32, H=8, T=1024, D=128: P = softmax(scale Q K^T) (bf16; the
                scores in binary32 on chip, the bits of bmm + softmax), O = P V (fp32)
  * decode  bf16  q [256, 32, 64], K, V [256, 32, 8192, 64], 2048-token chunks -> fp32
  * mm      fp32  X [200, 4096] @ W [4096, 256]
The headline `value` is the addmm GEMM throughput in TFLOP/s (algorithmic
2*M*N*K flops over the kernel's mean duration in the timed steps).  Every
operation is timed by HIP events that the runtime records at the start of
its first kernel and the end of its last (bi_set_launch_events attaches
them to the library's own dispatches).
Decode attention reports algorithmic HBM GB/s.  A
bitwise batch-invariance check (row 0 of the GEMM at M=1 vs M=8192, request
0 of decode at B=1 vs B=256) runs outside the timed region.  The CPU
baseline is the reference oracle timed on a bounded row sample of the
addmm workload on the host cores.

Prints one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

ADDMM = dict(M=8192, K=4096, N=14336)
CONV_B = 32
ATT = dict(B=32, H=8, T=1024, D=128)
DEC = dict(B=256, H=32, S=8192, D=64)
MM32 = dict(M=200, K=4096, N=256)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=2.0,
                    help="target host time of each leg (workload x thread count) of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma-separated subset of the step's operations (addmm, conv2d, attention, decode, "
                         "mm_fp32) to run, with no untimed extras and no CPU baseline: for profiler runs")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "gemm_bf16_addmm_M8192_traffic.txt"),
                    help="HBM-side bytes per GEMM launch measured with rocprofv3 counters")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (every operation would shard by "
              "request, head or output tile with no exchange between GPUs).", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from invariant_persistent_bf16_amd import bi, bi_bench

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bi.lib()
    print(f"# device: {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)

    known = ("addmm", "conv2d", "attention", "decode", "mm_fp32")
    only = [n for n in args.only.split(",") if n]
    for n in only:
        if n not in known:
            print(f"--only: unknown operation {n}; choose from {', '.join(known)}", file=sys.stderr)
            sys.exit(2)
    want = lambda n: not only or n in only

    # ------------------------------------------------ inputs (resident in HBM)
    W, bias, x0 = synth.addmm_shared()
    Wd, bd = W.to(dev), bias.to(dev)
    X = synth.addmm_batch(x0, ADDMM["M"], device=dev)
    Y = torch.empty(ADDMM["M"], ADDMM["N"], dtype=torch.bfloat16, device=dev)

    cw, cb, cx0 = synth.conv_shared()
    cwd, cbd = cw.to(dev), cb.to(dev)
    cx = synth.conv_batch(cx0, CONV_B, device=dev)
    cy = torch.empty(CONV_B, 1152, 16, 16, dtype=torch.bfloat16, device=dev)
    cws = torch.empty(bi.bi_conv2d_workspace_bytes(cx.shape, cw.shape, (14, 14)), dtype=torch.uint8,
                      device=dev)

    G = ATT["B"] * ATT["H"]
    att_scale = float(torch.tensor(1 / math.sqrt(ATT["D"]), dtype=torch.float32))
    Q = Kt = V = Pb = Ob = None
    if want("attention"):
        Q, Kt, V = synth.attn_batch(synth.attn_shared(), ATT["B"], device=dev)
        Pb = torch.empty(G, ATT["T"], ATT["T"], dtype=torch.bfloat16, device=dev)
        Ob = torch.empty(G, ATT["T"], ATT["D"], dtype=torch.float32, device=dev)

    dq = dk = dv = dout = dws = None
    if want("decode"):
        dq0 = synth.decode_shared()
        dq, dk, dv = synth.decode_batch(dq0, DEC["B"], device=dev)
        dout = torch.empty(DEC["B"], DEC["H"], DEC["D"], dtype=torch.float32, device=dev)
        dws = torch.empty(bi.bi_decode_attn_workspace_bytes(DEC["B"], DEC["H"], DEC["S"], DEC["D"]) // 4,
                          dtype=torch.float32, device=dev)

    mW, mX = synth.mm_inputs(Ms=(MM32["M"],))
    mWd, mXd = mW.to(dev), mX[MM32["M"]].to(dev)
    mY = torch.empty(MM32["M"], MM32["N"], dtype=torch.float32, device=dev)

    # A plain device copy of known size, so HBM counters can be calibrated
    # against it in a profiler run of this same command.
    calib_src = torch.empty(256 << 20, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    del calib_src, calib_dst
    torch.cuda.synchronize()

    ops = {
        "addmm": lambda: bi.bi_addmm(bd, X, Wd, out=Y),
        "conv2d": lambda: bi.bi_conv2d(cx, cwd, cbd, stride=(14, 14), out=cy, workspace=cws),
        # P = softmax(scale Q K^T) in one kernel (the bits of bmm + softmax, S
        # never written), then O = P V
        "attention": lambda: (bi.bi_attention_probs(Q, Kt, att_scale, out=Pb), bi.bi_bmm(Pb, V, out=Ob)),
        "decode": lambda: bi.bi_decode_attn(dq, dk, dv, 0.125, out=dout, workspace=dws),
        "mm_fp32": lambda: bi.bi_mm(mXd, mWd, out=mY),
    }
    names = only or list(ops)

    # Each operation is timed by events that its own kernels record (the
    # first kernel's start, the last kernel's end: bi_set_launch_events), so
    # neither event packets nor the gap before the first kernel are counted.
    def step(events=None):
        for i, n in enumerate(names):
            if events is not None:
                bi.bi_set_launch_events(*events[i])
            ops[n]()
        if events is not None:
            bi.bi_set_launch_events(None, None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in names] for _ in range(args.steps)]
    for es in ev:                 # create the events before the timed region
        for a, b in es:
            a.record()
            b.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms = {n: sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)) / args.steps
          for i, n in enumerate(names)}

    flops = {
        "addmm": 2.0 * ADDMM["M"] * ADDMM["N"] * ADDMM["K"],
        "conv2d": 2.0 * CONV_B * 1152 * 256 * 588,
        "attention": 2.0 * 2 * G * ATT["T"] * ATT["T"] * ATT["D"],
        "decode": 2.0 * 2 * DEC["B"] * DEC["H"] * DEC["S"] * DEC["D"],
        "mm_fp32": 2.0 * MM32["M"] * MM32["N"] * MM32["K"],
    }
    bytes_ = {
        "addmm": 2.0 * (ADDMM["M"] * ADDMM["K"] + ADDMM["K"] * ADDMM["N"] + ADDMM["N"] +
                        ADDMM["M"] * ADDMM["N"]),
        "conv2d": 2.0 * (CONV_B * 3 * 224 * 224 + 1152 * 588 + 1152 + CONV_B * 1152 * 256),
        # Q, K, V read, P written and read back (bf16), O written (fp32)
        "attention": G * (3 * ATT["T"] * ATT["D"] * 2 + ATT["T"] * ATT["T"] * (2 + 2) +
                          ATT["T"] * ATT["D"] * 4),
        "decode": DEC["B"] * DEC["H"] * (2 * DEC["S"] * DEC["D"] * 2 + DEC["D"] * 2 + DEC["D"] * 4),
        "mm_fp32": 4.0 * (MM32["M"] * MM32["K"] + MM32["K"] * MM32["N"] + MM32["M"] * MM32["N"]),
    }
    detail = {}
    for n in names:
        t = ms[n] * 1e-3
        detail[n] = {"ms": round(ms[n], 5), "TFLOP/s": round(flops[n] / t / 1e12, 2),
                     "GB/s": round(bytes_[n] / t / 1e9, 1)}
    if "addmm" in ms:
        detail["addmm"]["frac_bf16_peak"] = round(flops["addmm"] / (ms["addmm"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    if "decode" in ms:
        detail["decode"]["frac_hbm_peak"] = round(bytes_["decode"] / (ms["decode"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    if "mm_fp32" in ms:
        detail["mm_fp32"]["frac_fp32_mfma_peak"] = round(
            flops["mm_fp32"] / (ms["mm_fp32"] * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4)
    if only:
        # profiler runs: the timings of the selected operations only
        tf = flops["addmm"] / (ms["addmm"] * 1e-3) / 1e12 if "addmm" in ms else None
        print(json.dumps({"metric": "batch-invariant GEMM TFLOP/s & % bf16 MFMA peak; decode-attn GB/s; "
                                    "bitwise match", "value": None if tf is None else round(tf, 2),
                          "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "only": only, "ops": detail}), flush=True)
        return

    # ------------------------------------------- bitwise invariance (untimed)
    y1 = bi.bi_addmm(bd, X[:1], Wd)
    dq1, dk1, dv1 = dq[:1], dk[:1], dv[:1]
    o1 = bi.bi_decode_attn(dq1, dk1, dv1, 0.125)
    torch.cuda.synchronize()
    bit_gemm = torch.equal(y1[0].view(torch.int16), Y[0].view(torch.int16))
    bit_dec = torch.equal(o1[0].view(torch.int32), dout[0].view(torch.int32))
    invariance_records = {"addmm_row0_M1_vs_M8192": comparison_record(Y[:1], y1),
                          "decode_req0_B1_vs_B256": comparison_record(dout[:1], o1)}

    tflops = flops["addmm"] / (ms["addmm"] * 1e-3) / 1e12
    dec_gbs = bytes_["decode"] / (ms["decode"] * 1e-3) / 1e9
    traffic = gemm_traffic(args.traffic)

    out = {
        "metric": "batch-invariant GEMM TFLOP/s & % bf16 MFMA peak; decode-attn GB/s; bitwise match",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes of the pages' workloads)",
        "config": {"workload": "addmm bf16 M=8192 K=4096 N=14336 (+bias, bf16 out); one step also runs "
                               "conv2d SigLIP B=32, attention B=32 H=8 T=1024 D=128, decode B=256 H=32 "
                               "S=8192 D=64, mm fp32 M=200 K=4096 N=256",
                   "global_batch": ADDMM["M"], "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "roofline_decode": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4)},
        "decode_attn_GBps": round(dec_gbs, 1),
        "bitwise_match": {"addmm_row0_M1_vs_M8192": bool(bit_gemm),
                          "decode_req0_B1_vs_B256": bool(bit_dec)},
        "comparison": {"invariance": invariance_records},
        "ops": detail,
    }

    out["invariance_cost"] = invariance_cost(Wd, bd, x0, dq, dk, dv, Y)
    out["small_batch"] = small_batch(Wd, bd, x0, cwd, cbd, cx0)
    out["row_ops"] = row_ops(X, Y)
    out["paged_decode"] = paged_decode(dq, dk, dv, dout)
    out["prefill"] = prefill()
    out["f16_addmm"] = f16_addmm(W, bias, X, Y)

    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(args.cpu_seconds, dict(W=W, bias=bias, x0=x0, Wd=Wd, bd=bd, X=X),
                                   dict(cw=cw, cb=cb, cx=cx, cy_dev=None, cwd=cwd, cbd=cbd),
                                   dict(Q=Q, K=Kt, V=V, O=Ob, scale=att_scale),
                                   dict(q=dq, k=dk, v=dv, out=dout), dict(W=mW, X=mX[MM32["M"]], Y=mY))
        out["cpu_baseline"] = cpu
        out["comparison"]["oracle_parity_sample"] = parity
    del X, Y, Q, Kt, V, Pb, Ob, dq, dk, dv
    torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def comparison_record(got, ref):
    """The comparison figures of the VLA page's tracer ("Batch-Invariant
    VLAs", section "Profiling batch-invariance") between two device tensors
    whose first axis is the sample: max_abs_diff, mean_abs_diff, rmse,
    relative_l2_mean / _max (per sample, then mean and max over samples),
    output_abs_max (of got)."""
    import torch
    g = got.double().reshape(got.shape[0], -1)
    r = ref.double().reshape(ref.shape[0], -1).to(g.device)
    d = g - r
    nr = r.norm(dim=1)
    rel = d.norm(dim=1) / torch.where(nr > 0, nr, torch.ones_like(nr))
    return {"samples": int(g.shape[0]), "max_abs_diff": float(d.abs().max()),
            "mean_abs_diff": float(d.abs().mean()), "rmse": float(d.pow(2).mean().sqrt()),
            "relative_l2_mean": float(rel.mean()), "relative_l2_max": float(rel.max()),
            "output_abs_max": float(g.abs().max())}


def _time_ms(fn, iters=20):
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def _graph_us(fn, n=20):
    """GPU time of one call in microseconds, without the host's launch cost:
    n calls captured in a HIP graph (the library's kernels only, no memset
    nodes), replayed; best of 3 replays."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(3):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / n)
    del g
    return best


def _graph_us_seq(fns, reps=4):
    """GPU time per call of the calls fns[0], fns[1], ... captured in order
    (reps times over) in one graph and replayed: rotating operand copies gives
    the cold-cache rate of a working set larger than the 256 MB cache."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            for f in fns:
                f()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(3):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / (reps * len(fns)))
    del g
    return best


def small_batch(Wd, bd, x0, cwd, cbd, cx0):
    """Untimed extra: small batches of the addmm, conv and decode workloads,
    where 256x256 tiles (or one request's chunks) leave most compute units
    idle.  The library then picks the small-tile or 128-row kernels (same
    bits); forced 256x256 persistent-kernel times beside them.  GPU time from
    graph replay: warm (the same operands every call; a 117 MB W or a 64 MiB
    request stays in the 256 MB cache) and cold (3 W copies, 5 KV copies
    rotating)."""
    import torch

    import synth
    from invariant_persistent_bf16_amd import bi, bi_bench

    dev = Wd.device
    K, N = ADDMM["K"], ADDMM["N"]
    res = {}
    # Three copies of W (352 MB) rotate for the cold rate: one W fits the cache.
    Wcopies = [Wd] + [Wd.clone() for _ in range(2)]
    for M in (1, 64, 200):
        X = synth.addmm_batch(x0, M, device=dev)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        ta = _graph_us(lambda: bi.bi_addmm(bd, X, Wd, out=y))
        tc = _graph_us_seq([lambda W=W: bi.bi_addmm(bd, X, W, out=y) for W in Wcopies])
        tp = _graph_us(lambda: bi_bench.gemm_tile(X, Wd, 0, bias=bd, out=y))
        res[f"addmm_M{M}"] = {"us": round(ta, 2), "cold_us": round(tc, 2),
                              "tile_rows": bi_bench.gemm_tile_rows(1, M, N, K),
                              "persistent_us": round(tp, 2),
                              "W_GBps": round(K * N * 2 / (ta * 1e-6) / 1e9, 1),
                              "W_GBps_cold": round(K * N * 2 / (tc * 1e-6) / 1e9, 1)}
    del Wcopies
    cx = synth.conv_batch(cx0, 1, device=dev)
    cy = torch.empty(1, 1152, 16, 16, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(bi.bi_conv2d_workspace_bytes(cx.shape, cwd.shape, (14, 14)), dtype=torch.uint8, device=dev)
    tc = _graph_us(lambda: bi.bi_conv2d(cx, cwd, cbd, stride=(14, 14), out=cy, workspace=ws))
    # The conv's GEMM alone: packed weight [1152, 592] x unfold [256, 592]^T, row bias.
    Ap = torch.zeros(1152, 592, dtype=torch.bfloat16, device=dev)
    Ap[:, :588] = cwd.reshape(1152, 588)
    U = torch.zeros(256, 592, dtype=torch.bfloat16, device=dev)
    U[:, :588] = cx.reshape(3, 16, 14, 16, 14).permute(1, 3, 0, 2, 4).reshape(256, 588)
    yg = torch.empty(1152, 256, dtype=torch.bfloat16, device=dev)
    tg = {r: _graph_us(lambda: bi_bench.gemm_tile(Ap, U.t(), r, bias=cbd, bias_rows=True, out=yg))
          for r in (0, bi_bench.gemm_tile_rows(1, 1152, 256, 592))}
    res["conv2d_B1"] = {"us": round(tc, 2), "gemm_tile_rows": bi_bench.gemm_tile_rows(1, 1152, 256, 592),
                        "gemm_us": round(min(v for r, v in tg.items() if r != 0), 2),
                        "gemm_persistent_us": round(tg[0], 2)}
    H, S, D = DEC["H"], DEC["S"], DEC["D"]
    q1 = torch.randn(1, H, D, device=dev).to(torch.bfloat16)
    kv = [(torch.randn(1, H, S, D, device=dev).to(torch.bfloat16), torch.randn(1, H, S, D, device=dev).to(torch.bfloat16))
          for _ in range(5)]
    o1 = torch.empty(1, H, D, dtype=torch.float32, device=dev)
    ws1 = torch.empty(bi.bi_decode_attn_workspace_bytes(1, H, S, D) // 4 + 1, dtype=torch.float32, device=dev)
    tw = _graph_us(lambda: bi.bi_decode_attn(q1, kv[0][0], kv[0][1], 0.125, out=o1, workspace=ws1))
    tcd = _graph_us_seq([lambda k=k, v=v: bi.bi_decode_attn(q1, k, v, 0.125, out=o1, workspace=ws1) for k, v in kv])
    nb = 2 * H * S * D * 2
    res["decode_B1"] = {"us": round(tw, 2), "cold_us": round(tcd, 2), "GBps": round(nb / (tw * 1e-6) / 1e9, 1),
                        "GBps_cold": round(nb / (tcd * 1e-6) / 1e9, 1)}
    del kv
    return res


def invariance_cost(Wd, bd, x0, dq, dk, dv, Y):
    """Untimed extra: the invariant kernels against batch-size-tuned variants
    (split-K for the GEMM filling the CUs; for decode the handbook's split-KV
    by load and a fair split-KV whose parts fill the CUs and are merged in the
    same launch) at the batch sizes where they differ (GPU time from graph
    replay), plus an HBM read-rate probe."""
    import torch

    import synth
    from invariant_persistent_bf16_amd import bi, bi_bench

    dev = Wd.device
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    res = {"addmm": {}, "decode": {}}
    K, N = ADDMM["K"], ADDMM["N"]
    for M in (1, 64, 200, 2048):
        X = synth.addmm_batch(x0, M, device=dev)
        s = bi_bench.splitk_policy(M, N, K, 0)
        ws = torch.empty(max(1, s * M * N), dtype=torch.float32, device=dev)
        yv = Y[:M]
        ti = _graph_us(lambda: bi.bi_addmm(bd, X, Wd, out=yv)) * 1e-3
        ts = _graph_us(lambda: bi_bench.addmm_splitk(bd, X, Wd, s, out=yv, workspace=ws)) * 1e-3
        res["addmm"][str(M)] = {"invariant_us": round(ti * 1e3, 2), "splitk_us": round(ts * 1e3, 2),
                                "splits": s, "invariant_over_splitk": round(ti / ts, 3)}
    H, S, D = DEC["H"], DEC["S"], DEC["D"]
    for B in (1, 16, 64):
        q, k, v = dq[:B], dk[:B], dv[:B]
        s = bi_bench.decode_splits_policy(B, cus)
        o = torch.empty(B, H, D, dtype=torch.float32, device=dev)
        ws = torch.empty(bi_bench.lib().bi_bench_decode_attn_splits_workspace_bytes(B, H, S, D, s) // 4 + 1,
                         dtype=torch.float32, device=dev)
        wsf = torch.empty(bi.bi_decode_attn_workspace_bytes(B, H, S, D) // 4 + 1, dtype=torch.float32,
                          device=dev)
        tf = _graph_us(lambda: bi.bi_decode_attn(q, k, v, 0.125, out=o, workspace=wsf)) * 1e-3
        tl = _graph_us(lambda: bi_bench.decode_attn_splits(q, k, v, 0.125, s, out=o, workspace=ws)) * 1e-3
        # the fair competitor: parts sized to fill the CUs, waves sized to the
        # parts, merged in the same launch
        sk = bi_bench.decode_splitkv_policy(B, H, S, cus)
        wsk = bi_bench.decode_splitkv_workspace(B, H, D, sk, dev)
        tk = _graph_us(lambda: bi_bench.decode_attn_splitkv(q, k, v, 0.125, sk, wsk, out=o)) * 1e-3
        gbs = B * H * 2 * S * D * 2 / 1e9
        res["decode"][str(B)] = {"fixed_chunk_us": round(tf * 1e3, 2), "by_load_us": round(tl * 1e3, 2),
                                 "splits_by_load": s, "fixed_GBps": round(gbs / (tf * 1e-3), 1),
                                 "fixed_over_by_load": round(tf / tl, 3),
                                 "splitkv_fair_us": round(tk * 1e3, 2), "splitkv_fair_splits": sk,
                                 "fixed_over_splitkv_fair": round(tf / tk, 3)}
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    tp = _time_ms(lambda: bi_bench.read_probe(dk, sink), iters=5)
    res["hbm_read_probe_GBps"] = round(dk.numel() * 2 / (tp * 1e-3) / 1e9, 1)
    # The request shape of a GEMM's operand copies: 512 MiB of the KV buffer
    # read as 2 KiB rows in tiles of 256 rows, 64 or 128 bytes per row
    # and step (one K step of a 16-bit row, or a pair of steps).
    nb = 512 << 20
    buf = dk.view(-1)[: nb // dk.element_size()]
    res["row_step_read_GBps"] = {
        str(b): round(nb / (_time_ms(lambda b=b: bi_bench.row_step_read(buf, b, sink), iters=5) * 1e-3) / 1e9, 1)
        for b in (64, 128)}
    return res


def row_ops(X, Y):
    """Untimed extra (outside the step): the row operations beside the matmul on
    the LLM shapes of the addmm workload, against the HBM roofline: RMSNorm and
    mean over X [8192, 4096] bf16, log-softmax over the addmm output
    [8192, 14336] bf16 -> fp32 (bytes = input + output + weight).  "us": the
    same operands every call, so a 64 MB X and RMSNorm's output stay in the
    256 MB cache and the rate counts cache-served bytes; "cold_us": graph
    replay over copies of the operands that rotate (5 x 64 MB for RMSNorm and
    mean, 2 x 235 MB for log-softmax), each call's operands evicted by the
    others, the rate out of HBM."""
    import torch

    from invariant_persistent_bf16_amd import bi

    M, K, N = ADDMM["M"], ADDMM["K"], ADDMM["N"]
    w = torch.ones(K, dtype=torch.bfloat16, device=X.device)
    yr = torch.empty_like(X)
    ym = torch.empty(M, dtype=torch.float32, device=X.device)
    ys = torch.empty(M, N, dtype=torch.float32, device=X.device)
    xs = [X] + [X.clone() for _ in range(4)]
    yrs = [yr] + [torch.empty_like(X) for _ in range(4)]
    Ys = [Y, Y.clone()]
    cases = {
        "rms_norm_bf16_8192x4096": (lambda: bi.bi_rms_norm(X, w, 1e-6, out=yr),
                                    [lambda x=x, y=y: bi.bi_rms_norm(x, w, 1e-6, out=y) for x, y in zip(xs, yrs)],
                                    2 * M * K * 2 + 2 * K),
        "mean_bf16_8192x4096": (lambda: bi.bi_mean_rows(X, out=ym),
                                [lambda x=x: bi.bi_mean_rows(x, out=ym) for x in xs], 2 * M * K + 4 * M),
        "log_softmax_bf16_to_fp32_8192x14336": (lambda: bi.bi_log_softmax_rows(Y, out=ys),
                                                [lambda y=y: bi.bi_log_softmax_rows(y, out=ys) for y in Ys],
                                                M * N * (2 + 4)),
    }
    res = {}
    for name, (fn, fns, nbytes) in cases.items():
        t = _time_ms(fn, iters=50)
        tc = _graph_us_seq(fns)
        gbs = nbytes / (t * 1e-3) / 1e9
        gbc = nbytes / (tc * 1e-6) / 1e9
        res[name] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                     "cold_us": round(tc, 2), "GB/s_cold": round(gbc, 1),
                     "frac_hbm_peak_cold": round(gbc / PEAK_HBM_GBS, 4)}
    del yr, ym, ys, xs, yrs, Ys
    return res


def paged_decode(dq, dk, dv, dout):
    """Untimed extra: decode over a paged cache (16-token pages [num_pages, 32,
    16, 64], placed by a seeded permutation) holding the decode workload's K and
    V.  All requests at 8192 tokens (bits checked against the contiguous
    result), then seeded lengths uniform in [1, 8192]; bytes = the K and V rows
    of each request's tokens + q + out."""
    import torch

    from invariant_persistent_bf16_amd import bi

    dev = dq.device
    B, H, S, D = dk.shape
    P = 16
    npb = S // P
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    perm = torch.randperm(B * npb, generator=g, device=dev)
    kc = torch.empty(B * npb, H, P, D, dtype=dk.dtype, device=dev)
    vc = torch.empty_like(kc)
    kc[perm] = dk.view(B, H, npb, P, D).permute(0, 2, 1, 3, 4).reshape(B * npb, H, P, D)
    vc[perm] = dv.view(B, H, npb, P, D).permute(0, 2, 1, 3, 4).reshape(B * npb, H, P, D)
    bt = perm.view(B, npb).to(torch.int32)
    ws = torch.empty(bi.bi_decode_attn_paged_workspace_bytes(B, H, S, D) // 4, dtype=torch.float32, device=dev)
    o = torch.empty_like(dout)
    full = torch.full((B,), S, dtype=torch.int32, device=dev)
    lens = torch.randint(1, S + 1, (B,), generator=torch.Generator().manual_seed(22), dtype=torch.int32)
    res = {}
    for name, sl in (("all_8192", full), ("uniform_1_8192", lens.to(dev))):
        fn = lambda: bi.bi_decode_attn_paged(dq, kc, vc, bt, sl, S, 0.125, out=o, workspace=ws)
        t = _time_ms(fn)
        tokens = int(sl.sum().item())
        nbytes = tokens * H * D * 2 * 2 + B * H * D * (2 + 4)
        gbs = nbytes / (t * 1e-3) / 1e9
        res[name] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                     "mean_len": round(tokens / B, 1)}
        if name == "all_8192":
            fn()
            torch.cuda.synchronize()
            res[name]["bits_equal_contiguous"] = bool(torch.equal(o.view(torch.int32), dout.view(torch.int32)))
    del kc, vc
    return res


def f16_addmm(W, bias, X, Y):
    """Untimed extra: the fp16 configuration of the same addmm (M=8192, K=4096,
    N=14336, fp16 operands and output; the workload's values converted to
    fp16), timed in alternating blocks of 20 calls with the bf16 addmm on the
    same shape, after a warm-up of both, so that the two see the same clock
    and power state; the best block of each is reported."""
    import torch

    from invariant_persistent_bf16_amd import bi

    dev = X.device
    Wh, bh, Xh = W.to(dev, torch.float16), bias.to(dev, torch.float16), X.to(torch.float16)
    Wb, bb = W.to(dev), bias.to(dev)
    Yh = torch.empty(Y.shape, dtype=torch.float16, device=dev)
    f16 = lambda: bi.bi_addmm(bh, Xh, Wh, out=Yh, out_dtype=bi.BI_F16)
    b16 = lambda: bi.bi_addmm(bb, X, Wb, out=Y)
    for _ in range(10):
        f16()
        b16()
    t16, tb = float("inf"), float("inf")
    for _ in range(4):
        t16 = min(t16, _time_ms(f16, iters=20))
        tb = min(tb, _time_ms(b16, iters=20))
    M, K, N = ADDMM["M"], ADDMM["K"], ADDMM["N"]
    fl = 2 * M * N * K
    del Wh, Xh, Yh
    return {"ms": round(t16, 4), "TFLOP/s": round(fl / (t16 * 1e-3) / 1e12, 1),
            "frac_f16_peak": round(fl / (t16 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "bf16_same_blocks_ms": round(tb, 4),
            "bf16_same_blocks_frac_peak": round(fl / (tb * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def prefill():
    """Untimed extra: causal prefill attention over a paged cache (KV split at
    4096 tokens), one 8192-token prompt, 32 heads, D = 128, 16-token pages;
    flops = 4 * D * H * T(T+1)/2 (the two products over the causal pairs; the
    second product's two bfloat16 terms of P are not counted)."""
    import torch

    import synth
    from invariant_persistent_bf16_amd import bi

    T, H, D = 8192, 32, 128
    dev = torch.device("cuda:0")
    q, cu, p0, kc, vc, bt = synth.paged_prefill_inputs([0], [T], H=H, D=D, P=16, seed=31, device=dev)
    o = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(bi.bi_prefill_attn_paged_workspace_bytes(T, H, T, D) // 4, dtype=torch.float32, device=dev)
    t = _time_ms(lambda: bi.bi_prefill_attn_paged(q, cu, p0, T, kc, vc, bt, T, 1 / math.sqrt(D), out=o,
                                                  out_dtype=bi.BI_BF16, workspace=ws), iters=10)
    flops = 4 * D * H * T * (T + 1) / 2
    tf = flops / (t * 1e-3) / 1e12
    del q, kc, vc, o, ws
    return {"config": "B=1 T=8192 H=32 D=128 P=16 causal, bf16 out", "us": round(t * 1e3, 1),
            "TFLOP/s": round(tf, 1), "frac_bf16_peak": round(tf / (PEAK_BF16_TFLOPS), 4)}


def gemm_traffic(path):
    """Counter-measured bytes per GEMM launch, or None if the kernel source
    changed since the counters were taken (or no record exists)."""
    try:
        rec = dict(line.split(":", 1) for line in open(path) if ":" in line and not line.startswith("#"))
        if gemm_code_hash() != rec["source_sha256"].strip():
            return None
        return int(rec["bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def gemm_code_hash():
    """sha256 of the GEMM kernel's code lines (gemm_bf16.hpp + common.hpp,
    // comments and blank lines dropped), so that only a code change voids a
    stored counter record."""
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm_bf16.hpp", "common.hpp"):
        for line in open(os.path.join(ROOT, "invariant_persistent_bf16_amd", "csrc", f), encoding="utf-8"):
            code = line.split("//", 1)[0].strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_units(fn, units, target_s, first=1):
    """Run fn(list of unit indices) on growing batches of units until about
    target_s seconds of host time; returns (units done, seconds, outputs)."""
    done, t, n, outs = 0, 0.0, first, []
    while done < len(units) and (t < target_s or done == 0):
        sel = units[done:done + n]
        t0 = time.perf_counter()
        outs.append((sel, fn(sel)))
        t += time.perf_counter() - t0
        done += len(sel)
        if t < target_s:
            per = t / done
            n = max(1, min(len(units) - done, int((target_s - t) / per * 0.6)))
    return done, t, outs


def cpu_baseline(target_s, addmm, conv, att, dec, mm32):
    """The fp64 oracle (test infrastructure, as it stands) timed on the host,
    per workload, at one thread and at all of the host's threads, each on a
    bounded sample of about target_s seconds: rows of the addmm, images of the
    convolution, slices of the attention, requests of the decode, and the
    whole binary32 mm.  Each leg reports its units, the seconds, the oracle's
    rate in the workload's unit, and a labelled linear extrapolation of the
    host time to the full workload.  Also returns the comparison record of the
    GPU's outputs on the all-core addmm sample and decode sample against the
    oracle (GPU rows recomputed alone: by row invariance the same bits)."""
    import numpy as np
    import torch

    import oracle
    from invariant_persistent_bf16_amd import bi

    dev = addmm["Wd"].device
    all_threads = oracle.set_threads()
    res = {"cpu_model": _cpu_model(), "host_threads": all_threads, "legs": {}}
    g = torch.Generator().manual_seed(4242)

    def order(n):
        return [0] + (torch.randperm(n - 1, generator=g) + 1).tolist()

    M, K, N = ADDMM["M"], ADDMM["K"], ADDMM["N"]
    Xh = addmm["X"].cpu()
    G = ATT["B"] * ATT["H"]
    T, Dh = ATT["T"], ATT["D"]
    legs = {
        "addmm": (order(M), M, 2.0 * K * N, "row",
                  lambda sel: oracle.mm(Xh[sel], addmm["W"], addmm["bias"])),
        "conv2d": (order(CONV_B), CONV_B, 2.0 * 1152 * 256 * 588, "image",
                   lambda sel: oracle.conv2d_direct(conv["cx"][sel].cpu(), conv["cw"], conv["cb"], stride=(14, 14))),
        "attention": (order(G), G, 4.0 * T * T * Dh, "slice",
                      lambda sel: oracle.attention(att["Q"][sel].cpu(), att["K"][sel].cpu(), att["V"][sel].cpu(),
                                                   att["scale"], p_bf16=True)),
        "decode": (order(DEC["B"]), DEC["B"], 4.0 * DEC["H"] * DEC["S"] * DEC["D"], "request",
                   lambda sel: oracle.decode(dec["q"][sel].cpu(), dec["k"][sel].cpu(), dec["v"][sel].cpu(), 0.125)),
        "mm_fp32": ([0], 1, 2.0 * MM32["M"] * MM32["N"] * MM32["K"], "whole product",
                    lambda sel: oracle.mm(mm32["X"], mm32["W"])),
    }
    parity = {}
    try:
        for name, (units, total, flop_per_unit, unit_name, fn) in legs.items():
            res["legs"][name] = {}
            for threads in (1, all_threads):
                oracle.set_threads(threads)
                done, t, outs = _time_units(fn, units, target_s)
                rate = flop_per_unit * done / t
                res["legs"][name][f"threads_{threads}"] = {
                    "units": done, "unit": unit_name, "seconds": round(t, 3),
                    "GFLOP/s": round(rate / 1e9, 3),
                    "full_workload_seconds_extrapolated": round(t / done * total, 2)}
                if threads == all_threads and name in ("addmm", "decode"):
                    sel = [u for s_, _ in outs for u in s_]
                    ref = np.concatenate([o for _, o in outs])
                    if name == "addmm":
                        got = bi.bi_addmm(addmm["bd"], addmm["X"][sel], addmm["Wd"], out_dtype=bi.BI_F32)
                    else:
                        got = bi.bi_decode_attn(dec["q"][sel], dec["k"][sel], dec["v"][sel], 0.125)
                    torch.cuda.synchronize()
                    parity[name] = comparison_record(got, torch.from_numpy(ref))
                    parity[name]["units"] = sel[:8] + (["..."] if len(sel) > 8 else [])
    finally:
        oracle.set_threads(all_threads)
    a = res["legs"]["addmm"][f"threads_{all_threads}"]
    cpu = {"value": round(a["GFLOP/s"] / 1e3, 6), "unit": "TFLOP/s", "cores": all_threads, "kind": "oracle",
           "sample": f"{a['units']} rows of the addmm workload (K=4096, N=14336, fp64 loops), {a['seconds']} s; "
                     f"per-workload legs at 1 and {all_threads} threads below",
           "cpu_model": res["cpu_model"], "per_workload": res["legs"]}
    return cpu, parity


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the block-quantized decode weight stream on one MI355X.

One step = one decoded token's pass over a 27B-dense model's GEMV weight stream: 64 layers,
each q|k|v (7168 x 5120, the three projections stacked since they read the same input),
o (5120 x 5120), gate|up (34816 x 5120, stacked likewise) and down (5120 x 17408), all
Q4_0, batch 1, as ONE chain launch of the 256 GEMVs in layer order, each GEMV waiting
(device-wide) for all earlier ones, as a decode step's data dependencies require.  Weights
are seeded N(0, 0.02) draws quantized to Q4_0, inputs N(0, 1), all resident in HBM before
the timed region.  The headline is achieved HBM GB/s over the algorithmic bytes of the
stream (packed codes and scales read once, fp32 inputs read, outputs written) and the
equivalent decode tokens/s (1 / time per pass).  Reported beside it: the per-step median
and 10th/90th percentiles, the same GEMVs as one chain without waits (the streaming rate
alone), and each layer shape's sustained rate over 64 independent copies.

Other workloads (--workload): the single 4096 x 4096 GEMV, the Q8_0 stream at M = 1/4/8,
the 128-expert MoE layer through qmv_id, and the 512 x 5120 x 17408 prefill GEMM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA, published (POP/s = 5.0e15)
# Vector ALU rates of MI355X.  The published fp32 vector peak, 157.3 TFLOP/s = 256 CUs x
# 2.4 GHz x 128 FMA lanes per cycle x 2 flops, is the rate of plain fp32 FMAs: 78.65 T lane-ops
# per second.  Other vector operations (conversions, bit operations, packed binary16,
# mixed-precision FMAs) issue at 256 x 64 lanes x 2.4 GHz = 39.3 T lane-ops/s.  (Measured on
# the box with register-only loops: v_fmac_f32 / v_fma_f32 1.33-1.41 wave instructions per CU
# and cycle at 2.4 GHz, v_cvt_f32_i32 (SDWA), v_cvt_f32_ubyte, v_and_or_b32, v_pk_add_f16 and
# v_fma_mix_f32 0.81-0.90.)  An ALU roofline prices a kernel's algorithmic FMAs and other
# operations each at its rate; its 'achieved' figure is in FMA-equivalent lane-ops per second
# (an other operation counts as two) against the FMA peak.
FMA_PEAK_TOPS = 157.3 / 2
VALU_OTHER_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12


def alu_roofline(fma_ops, other_ops, seconds, kernel, launch_us, **extra):
    eq = (fma_ops + 2.0 * other_ops) / seconds / 1e12
    return {"bound": "alu", "achieved": round(eq, 3), "peak": round(FMA_PEAK_TOPS, 3),
            "unit": "T FMA-equivalent lane-op/s", "frac": round(eq / FMA_PEAK_TOPS, 4), "traffic": None,
            "kernel": kernel, "avg_launch_us": launch_us, **extra}


def alu_seconds(fma_ops, other_ops):
    return fma_ops / (FMA_PEAK_TOPS * 1e12) + other_ops / (VALU_OTHER_PEAK_TOPS * 1e12)


def binding_roofline(hbm_bytes, fma_ops, other_ops, seconds, kernel, launch_us, traffic):
    """The roofline that binds: HBM (algorithmic bytes at 8 TB/s) or the vector ALU (the
    algorithmic FMAs and conversions at their rates), whichever takes longer; both fractions
    (ideal time / measured time) beside it."""
    t_h = hbm_bytes / (HBM_PEAK_GBS * 1e9)
    t_a = alu_seconds(fma_ops, other_ops)
    gbs = hbm_bytes / seconds / 1e9
    if t_a > t_h:
        r = alu_roofline(fma_ops, other_ops, seconds, kernel, launch_us, hbm_gbs=round(gbs, 1))
        r["traffic"] = traffic
    else:
        r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
             "avg_launch_us": launch_us}
    r["hbm_frac"] = round(t_h / seconds, 4)
    r["alu_frac"] = round(t_a / seconds, 4)
    return r


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense27b_q4_0",
                    choices=["dense27b_q4_0", "dense27b_q8_0", "gemv4096", "moe", "prefill", "prefill_q4_0",
                             "prefill_moe"])
    ap.add_argument("--M", type=int, default=1, help="batch for dense27b_q8_0 (1, 4 or 8)")
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--no-graph", action="store_true", help="eager launches instead of a graph")
    ap.add_argument("--separate", action="store_true",
                    help="one launch per GEMV (graph replay) instead of one chain launch per token")
    ap.add_argument("--compare-separate", action="store_true",
                    help="also time the pass as separate launches (reported beside the chain)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------- inputs

def make_matrix(fmt, N, K, key, torch, gen, bqm):
    """Seeded Gaussian weights -> interchange blocks -> packed layout, all on the GPU."""
    w = gen.normal((N, K), key, std=0.02, device="cuda")
    wi = gen.encode_q4_0(w) if fmt == "q4_0" else gen.encode_q8_0(w)
    del w
    wp = bqm.repack(fmt, wi.reshape(-1), N, K)
    return wp


def weight_bytes(fmt, N, K):
    return N * (K // 32) * (18 if fmt == "q4_0" else 34)   # codes + scales, no padding


# --------------------------------------------------------------------- timing

def time_steps(run, steps, warmup, torch, use_graph):
    """Warm up, then time exactly `steps` steps between two synchronizations."""
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            run()                      # eager once (sets kernel attributes)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            run()
        step = g.replay
    else:
        step = run
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps   # ms per step


def step_percentiles(run, steps, torch):
    """Each of `steps` further steps bracketed by its own events: median, 10th and 90th
    percentile of the per-step time in ms."""
    cur = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(cur)
        run()
        b.record(cur)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"median": round(float(np.median(t)), 4), "p10": round(float(np.percentile(t, 10)), 4),
            "p90": round(float(np.percentile(t, 90)), 4), "n": int(steps)}


def chain_of(fmt, M, items, wait, torch, bqm):
    """Prepare chains over (w, N, K, x, y) items; returns the run function (the workspaces
    stay alive in its closure).  One chain when it can be planned; a chain without waits whose
    single segment leaves a workgroup more partial sums than its local memory holds (long K
    at M >= 4) is split into halves, run back to back."""
    descs = [bqm.gemv(fmt, w, x, y, N, K, wait=wait and i > 0, M=M) for i, (w, N, K, x, y) in enumerate(items)]
    ws = torch.zeros(bqm.chain_workspace_bytes(len(descs)), dtype=torch.uint8, device="cuda")
    try:
        bqm.bqm_chain_prepare(descs, ws)
    except bqm.BqmError as e:
        if e.status != 2 or wait or len(items) < 2:
            raise
        h = len(items) // 2
        parts = [chain_of(fmt, M, items[:h], False, torch, bqm), chain_of(fmt, M, items[h:], False, torch, bqm)]

        def run_parts():
            for r in parts:
                r()
        run_parts.ws = parts[0].ws
        run_parts.chains = sum(getattr(r, "chains", 1) for r in parts)
        return run_parts

    def run():
        bqm.qmv_chain(fmt, M, ws, len(descs))
    run.ws = ws
    run.chains = 1
    return run


def per_launch_ms(launches, torch, reps=3):
    """Average duration of each launch, bracketed by events on the stream it runs on.  A spin
    kernel ahead of them holds the stream while the host enqueues every launch and event, so
    that the launches run back to back and a bracket holds a launch's own time on the GPU
    rather than the host's submission of it to an idle queue (which added 20-30 us to a
    launch of about 125 us)."""
    cur = torch.cuda.current_stream()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in launches] for _ in range(reps)]
    torch.cuda.synchronize()
    # about 2.4e6 spin cycles per ms; 0.1 ms of host time per launch and its events, at
    # least 2 ms
    torch.cuda._sleep(int(2.4e6 * max(2.0, 0.1 * reps * len(launches))))
    for r in range(reps):
        for (a, b), fn in zip(ev[r], launches):
            a.record(cur)
            fn()
            b.record(cur)
    torch.cuda.synchronize()
    return np.array([sum(ev[r][i][0].elapsed_time(ev[r][i][1]) for r in range(reps)) / reps
                     for i in range(len(launches))])


def traffic_from_profiles(kernel_key):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        ent = d[kernel_key]
        src = os.path.join(ROOT, "block_quantized_matrix_amd", "csrc", ent["source"])
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != ent["source_sha256"]:
            return None
        return float(ent["hbm_bytes_per_launch"])
    except Exception:
        return None


# --------------------------------------------------------------------- CPU baseline

def cpu_baseline(fmt, shapes, key_of, seconds, torch, gen, unit="GB/s", M=1, limit=64, what="layers"):
    """The oracle (never tuned) on the host cores, on whole layers of the same stream until
    about `seconds` of work is done; rate in the metric's unit over the same bytes."""
    import oracle
    oracle.build(force=False)
    done_bytes, t_used, layers = 0, 0.0, 0
    while t_used < seconds and layers < limit:
        for name, N, K in shapes:
            wi = (gen.encode_q4_0 if fmt == "q4_0" else gen.encode_q8_0)(
                gen.normal((N, K), key_of(layers, name), std=0.02, device="cuda"))
            wh = wi.cpu().numpy()
            x = gen.normal((M, K), key_of(layers, name) + ("x",), device="cuda").cpu().numpy()
            t = time.perf_counter()
            oracle.qmv(fmt, wh, x, N, K)
            t_used += time.perf_counter() - t
            done_bytes += weight_bytes(fmt, N, K) + 4 * M * (K + N)
        layers += 1
    return {"value": round(done_bytes / t_used / 1e9, 4), "unit": unit, "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{layers} of the {limit} {what} ({len(shapes)} GEMVs each), full rows, "
                      f"{t_used:.1f} s of oracle time"}


def _host_blocks(fmt, N, K, key, gen):
    """Interchange blocks of the seeded weights (the same draws as make_matrix), on the host."""
    w = gen.normal((N, K), key, std=0.02, device="cuda")
    wi = gen.encode_q4_0(w) if fmt == "q4_0" else gen.encode_q8_0(w)
    del w
    return wi.cpu().numpy()


def cpu_baseline_moe(T, E, top_k, H, F, seconds, gen):
    """The oracle's expert-indexed GEMV (gate, up, down of one layer, the definition: every
    slot's rows in turn) on the host cores; GB/s over the same unique-expert and activation
    bytes as the GPU figure."""
    import oracle
    oracle.build(force=False)
    gate = _host_blocks("q4_0", E * F, H, ("moe", 0, "gate"), gen)
    up = _host_blocks("q4_0", E * F, H, ("moe", 0, "up"), gen)
    down = _host_blocks("q4_0", E * H, F, ("moe", 0, "down"), gen)
    ids = gen.router_ids(T, E, top_k, ("moe-ids", 0, T))
    x = gen.normal((T, H), ("moe-x", 0, T), device="cuda").cpu().numpy()
    xd = gen.normal((T, top_k, F), ("moe-xd", 0, T), device="cuda").cpu().numpy()
    uniq = len(np.unique(ids))
    per = uniq * (weight_bytes("q4_0", F, H) * 2 + weight_bytes("q4_0", H, F)) + \
        4 * (2 * T * H + 2 * T * top_k * F + T * top_k * F + T * top_k * H)
    done, t_used, reps = 0, 0.0, 0
    while t_used < seconds and reps < 64:
        t = time.perf_counter()
        oracle.qmv_id("q4_0", gate, E, F, H, ids, x, H, 0)
        oracle.qmv_id("q4_0", up, E, F, H, ids, x, H, 0)
        oracle.qmv_id("q4_0", down, E, H, F, ids, xd, top_k * F, F)
        t_used += time.perf_counter() - t
        done += per
        reps += 1
    return {"value": round(done / t_used / 1e9, 4), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"layer 0 of 8 at T = {T} (gate, up, down; {uniq} unique experts), "
                      f"{reps} passes, {t_used:.1f} s of oracle time"}


def cpu_baseline_qmm(fmt, M, N, K, key, xkey, seconds, gen):
    """The oracle's prefill product (int32 block sums, fp64 rescale) on the host cores over
    leading row ranges of the same weights, until about `seconds` of work; int8 TOP/s."""
    import oracle
    oracle.build(force=False)
    W = _host_blocks(fmt, N, K, key, gen).reshape(N, -1)
    X = gen.normal((M, K), xkey, device="cuda").cpu().numpy()
    Xq, dx = oracle.quantize_q8_act(X, K)   # the oracle's own quantizer
    fn = oracle.qmm_q4_0 if fmt == "q4_0" else oracle.qmm_q8_0
    rows, t_used, chunk = 0, 0.0, 64
    while t_used < seconds and rows < N:
        n = min(chunk, N - rows)
        t = time.perf_counter()
        fn(W[rows:rows + n], Xq, dx, n, K)
        t_used += time.perf_counter() - t
        rows += n
        chunk = min(4 * chunk, 1024)
    return {"value": round(2.0 * M * rows * K / t_used / 1e12, 6), "unit": "TOP/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"output columns 0..{rows - 1} of {N} (all {M} rows, K = {K}), "
                      f"{t_used:.1f} s of oracle time"}


def cpu_baseline_qmm_id(E, top_k, H, F, T, seconds, gen):
    """The oracle's expert-indexed prefill product (gate projection of layer 0) on the host
    cores, over the first rows of every expert, until about `seconds` of work; TOP/s of
    useful int8 products."""
    import oracle
    oracle.build(force=False)
    gate = _host_blocks("q4_0", E * F, H, ("moep", 0, "gate"), gen).reshape(E, F, -1)
    ids = gen.router_ids(T, E, top_k, ("moep-ids", 0))
    x = gen.normal((T, H), ("moep-x", 0), device="cuda").cpu().numpy()
    xq, xdx = oracle.quantize_q8_act(x, H)
    n, t_used = 8, 0.0
    while True:
        Wn = np.ascontiguousarray(gate[:, :n])
        t = time.perf_counter()
        oracle.qmm_id("q4_0", Wn, E, n, H, ids, xq, xdx, 1, 0)
        t_used = time.perf_counter() - t
        if t_used >= seconds / 4 or n >= F:
            break
        n = min(F, n * 4)
    return {"value": round(2.0 * T * top_k * n * H / t_used / 1e12, 6), "unit": "TOP/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"gate projection of layer 0, output rows 0..{n - 1} of {F} of every expert, "
                      f"all {T * top_k} slots, {t_used:.1f} s of oracle time"}


# --------------------------------------------------------------------- workloads

def run_dense(args, torch, gen, bqm, fmt="q4_0"):
    M = args.M if fmt == "q8_0" else 1
    shapes = gen.DENSE27B_FUSED_SHAPES
    qmv = bqm.qmv_q4_0 if fmt == "q4_0" else bqm.qmv_q8_0
    say(f"generating {args.layers} layers of {fmt} weights on the GPU ...")
    t = time.time()
    mats, xs, ys = [], [], []
    for l in range(args.layers):
        for name, N, K in shapes:
            mats.append((make_matrix(fmt, N, K, ("dense27b", fmt, l, name), torch, gen, bqm), N, K))
            xs.append(gen.normal((M, K), ("dense27b-x", l, name, M), device="cuda"))
            ys.append(torch.empty((M, N), device="cuda"))
    torch.cuda.synchronize()
    say(f"  done in {time.time() - t:.1f} s; {torch.cuda.memory_allocated() / 2**30:.2f} GiB resident")
    wbytes = sum(weight_bytes(fmt, N, K) for _, N, K in mats)
    abytes = sum(4 * M * (K + N) for _, N, K in mats)
    launches = [(lambda w=w, x=x, y=y, N=N, K=K: qmv(w, x, y, M, N, K))
                for (w, N, K), x, y in zip(mats, xs, ys)]

    def run_separate():
        for f in launches:
            f()

    total = wbytes + abytes
    per_bytes = np.array([weight_bytes(fmt, N, K) + 4 * M * (K + N) for _, N, K in mats])
    use_chain = not args.separate
    if use_chain:
        # one launch per token: the 256 GEMVs in layer order, each waiting (device-wide)
        # for all earlier ones, as a decode step's data dependencies require
        descs = [bqm.gemv(fmt, w, x, y, N, K, wait=i > 0, M=M)
                 for i, ((w, N, K), x, y) in enumerate(zip(mats, xs, ys))]
        ws = torch.zeros(bqm.chain_workspace_bytes(len(descs)), dtype=torch.uint8, device="cuda")
        bqm.bqm_chain_prepare(descs, ws)

        def run():
            bqm.qmv_chain(fmt, M, ws, len(descs))

        ms = time_steps(run, args.steps, args.warmup, torch, False)
        status = bqm.bqm_chain_status(ws)
        if status != 0:
            raise RuntimeError(f"chain reported error {status}")
        dur = per_launch_ms([run], torch, reps=max(3, args.steps // 2))
        achieved = total / (float(dur.mean()) * 1e-3) / 1e9
        # batches of 5-8 inputs run on the matrix-core form of the chain (every K here is a
        # multiple of 256)
        mc = M >= 5
        kernel = f"{'k_qmv_chain_mc' if mc else 'k_qmv_chain'} ({fmt.upper()}, M={M}, {len(descs)} GEMVs per launch)"
        launch_us = round(1e3 * float(dur.mean()), 3)
        kkey = f"qmv_chain_{fmt}_dense27b" if M == 1 else f"qmv_chain_{fmt}_m{M}_dense27b"
        pct = step_percentiles(run, max(20, args.steps), torch)
        # diagnostics beside the headline: the same GEMVs with no waits (the stream alone),
        # and each layer shape's sustained rate over its 64 independent copies
        items = [(w, N, K, x, y) for (w, N, K), x, y in zip(mats, xs, ys)]
        run_ind = chain_of(fmt, M, items, False, torch, bqm)
        ms_ind = time_steps(run_ind, args.steps, args.warmup, torch, False)
        per_shape = {}
        for j, (name, N, K) in enumerate(shapes):
            sub = items[j::len(shapes)]
            run_s = chain_of(fmt, M, sub, False, torch, bqm)
            ms_s = time_steps(run_s, max(5, args.steps // 2), 2, torch, False)
            b = sum(weight_bytes(fmt, N, K) + 4 * M * (N + K) for _ in sub)
            per_shape[f"{name} {N}x{K}"] = {"copies": len(sub), "ms": round(ms_s, 4),
                                             "gbs": round(b / (ms_s * 1e-3) / 1e9, 1)}
        if bqm.bqm_chain_status(run_ind.ws) != 0:
            raise RuntimeError("independent chain reported an error")
    else:
        ms = time_steps(run_separate, args.steps, args.warmup, torch, not args.no_graph)
        dur = per_launch_ms(launches, torch)
        achieved = per_bytes.sum() / (dur.sum() * 1e-3) / 1e9
        kernel = f"k_qmv ({fmt.upper()} M={M})"
        launch_us = round(1e3 * float(dur.mean()), 3)
        kkey = f"qmv_{fmt}_m{M}_dense27b"
    gbs = total / (ms * 1e-3) / 1e9
    say(f"step {ms:.3f} ms, {gbs:.1f} GB/s, {1e3 / ms:.1f} passes/s")
    # the same pass as separate launches (graph replay), for reference
    ms_sep = time_steps(run_separate, max(3, args.steps // 2), 1, torch, not args.no_graph) \
        if use_chain and args.compare_separate else (ms if not use_chain else None)
    traffic = traffic_from_profiles(kkey)
    res = {
        "metric": "Q4_0 GEMV achieved HBM GB/s (% of peak) + equiv 27B decode tok/s"
        if fmt == "q4_0" else f"Q8_0 GEMV (M={M}) achieved HBM GB/s + equiv 27B decode tok/s",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"27B-dense decode weight stream, {fmt.upper()}, batch {M}: "
                               f"{args.layers} layers x (qkv 7168x5120, o 5120x5120, "
                               f"gate_up 34816x5120, down 5120x17408)",
                   "layers": args.layers, "gemv_launches_per_step": len(mats),
                   "weight_bytes": wbytes, "activation_bytes": abytes,
                   "launch": "one chain launch per token" if use_chain else
                   ("HIP graph of separate launches" if not args.no_graph else "separate launches")},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "equiv_tok_s": round(1e3 / ms, 2),
        "separate_launches_ms_per_step": None if ms_sep is None else round(ms_sep, 4),
        **({"step_ms": pct,
            "independent_gemvs": {"ms_per_step": round(ms_ind, 4),
                                  "gbs": round(total / (ms_ind * 1e-3) / 1e9, 1),
                                  "chains": run_ind.chains,
                                  "note": "the same 256 GEMVs as chains without waits"},
            "per_shape_sustained": per_shape} if use_chain else {}),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": kernel, "avg_launch_us": launch_us},
    }
    # The vector-ALU ceiling: each weight takes at least M fp32 multiply-adds (one per input
    # row) and one code conversion.  Where that ceiling is below the HBM one it is the
    # binding roofline and is reported as such.  On the matrix-core form (batches 5-8) the
    # products run on the matrix cores, and the vector ALU converts each code once and applies
    # each block scale once per row and input (M / 32 multiply-adds per weight).
    nweights = sum(N * K for _, N, K in mats)
    mc = use_chain and M >= 5
    t_alu = alu_seconds(M * nweights / 32, nweights) if mc else alu_seconds(M * nweights, nweights)
    alu_ceiling_gbs = total / t_alu / 1e9
    res["alu_ceiling_gbs"] = round(alu_ceiling_gbs, 1)
    res["hbm_frac"] = round(achieved / HBM_PEAK_GBS, 4)
    launch_s = float(dur.mean() if use_chain else dur.sum()) * 1e-3
    res["alu_frac"] = round(t_alu / launch_s, 4)
    if alu_ceiling_gbs < HBM_PEAK_GBS:
        res["roofline"] = alu_roofline(M * nweights / 32 if mc else M * nweights, nweights, launch_s,
                                       kernel, launch_us, hbm_gbs=round(achieved, 1))
        res["roofline"]["traffic"] = traffic
    if fmt == "q8_0":
        res["equiv_tok_s_aggregate"] = round(M * 1e3 / ms, 2)
    if not args.no_cpu:
        say("timing the oracle on the host ...")
        res["cpu_baseline"] = cpu_baseline(fmt, shapes, lambda l, n: ("dense27b", fmt, l, n),
                                           args.cpu_seconds, torch, gen, M=M)
    return res


def run_gemv4096(args, torch, gen, bqm):
    """64 back-to-back Q4_0 GEMVs 4096 x 4096 over distinct weight copies (604 MB, more than
    twice the 256 MB last-level cache), as one chain launch without waits (they are
    independent); the same GEMVs as separate launches (graph replay) are reported beside."""
    N = K = 4096
    copies = 64
    mats = [make_matrix("q4_0", N, K, ("gemv4096", c), torch, gen, bqm) for c in range(copies)]
    x = gen.normal((1, K), ("gemv4096-x", 0), device="cuda")
    ys = [torch.empty((1, N), device="cuda") for _ in range(copies)]
    descs = [bqm.gemv("q4_0", w, x, y, N, K, wait=False) for w, y in zip(mats, ys)]
    ws = torch.zeros(bqm.chain_workspace_bytes(copies), dtype=torch.uint8, device="cuda")
    bqm.bqm_chain_prepare(descs, ws)

    def run():
        bqm.qmv_chain("q4_0", 1, ws, copies)

    ms = time_steps(run, args.steps, args.warmup, torch, False)
    if bqm.bqm_chain_status(ws) != 0:
        raise RuntimeError("chain reported an error")
    per = weight_bytes("q4_0", N, K) + 4 * (N + K)
    gbs = per * copies / (ms * 1e-3) / 1e9
    dur = per_launch_ms([run], torch, reps=max(3, args.steps // 2))
    achieved = per * copies / (float(dur.mean()) * 1e-3) / 1e9
    launches = [(lambda w=w, y=y: bqm.qmv_q4_0(w, x, y, 1, N, K)) for w, y in zip(mats, ys)]

    def run_sep():
        for f in launches:
            f()

    ms_sep = time_steps(run_sep, max(3, args.steps // 2), 1, torch, not args.no_graph)
    # single launches, as a caller makes them: 256 calls over the 64 copies, each bracketed
    # by its own events on the stream it runs on
    cur = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(256)]
    for i, (a, b) in enumerate(ev):
        a.record(cur)
        launches[i % copies]()
        b.record(cur)
    torch.cuda.synchronize()
    single = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3   # us
    single_stats = {"n": len(single), "median_us": round(float(np.median(single)), 2),
                    "p10_us": round(float(np.percentile(single, 10)), 2),
                    "p90_us": round(float(np.percentile(single, 90)), 2),
                    "gbs_at_median": round(per / (float(np.median(single)) * 1e-6) / 1e9, 1)}
    return {"metric": "Q4_0 GEMV 4096x4096 sustained GB/s", "value": round(gbs, 2), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": "Q4_0 GEMV 4096x4096 batch 1, 64 distinct weight copies per step",
                       "launch": "one chain launch of the 64 independent GEMVs"},
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "separate_launches_ms_per_step": round(ms_sep, 4),
            "separate_launches_gbs": round(per * copies / (ms_sep * 1e-3) / 1e9, 1),
            "single_launch": single_stats,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic_from_profiles("qmv_chain_q4_0_gemv4096"),
                         "kernel": "k_qmv_chain (Q4_0, M=1, 64 GEMVs per launch)",
                         "avg_launch_us": round(1e3 * float(dur.mean()), 3)},
            **({} if args.no_cpu else {"cpu_baseline": cpu_baseline(
                "q4_0", [("w", N, K)], lambda c, n: ("gemv4096", c), args.cpu_seconds, torch, gen,
                limit=copies, what="weight copies")})}


def run_moe(args, torch, gen, bqm):
    sh = gen.MOE_SHAPE
    E, top_k, H, F = sh["E"], sh["top_k"], sh["hidden"], sh["ffn"]
    n_layers = 8   # distinct MoE layers (8 x 1.36 GB) cycled so the expert weights stream HBM
    out = []
    for T in (1, 16):
        layers = []
        for l in range(n_layers):
            gate = make_matrix("q4_0", E * F, H, ("moe", l, "gate"), torch, gen, bqm)
            up = make_matrix("q4_0", E * F, H, ("moe", l, "up"), torch, gen, bqm)
            down = make_matrix("q4_0", E * H, F, ("moe", l, "down"), torch, gen, bqm)
            ids = torch.from_numpy(gen.router_ids(T, E, top_k, ("moe-ids", l, T))).cuda()
            x = gen.normal((T, H), ("moe-x", l, T), device="cuda")
            xd = gen.normal((T, top_k, F), ("moe-xd", l, T), device="cuda")
            yg = torch.empty((T, top_k, F), device="cuda")
            yu = torch.empty((T, top_k, F), device="cuda")
            yd = torch.empty((T, top_k, H), device="cuda")
            uniq = len(np.unique(ids.cpu().numpy()))
            layers.append((gate, up, down, ids, x, xd, yg, yu, yd, uniq))
        # router weights and the layer outputs of the down projection with the weighted sum
        rws = [torch.from_numpy(gen.router_weights(T, top_k, ("moe-w", l, T))).cuda() for l in range(n_layers)]
        youts = [torch.empty((T, H), device="cuda") for _ in range(n_layers)]

        def run():
            for gate, up, down, ids, x, xd, yg, yu, yd, _ in layers:
                bqm.qmv_id("q4_0", gate, E, F, H, ids, T, top_k, x, H, 0, yg)
                bqm.qmv_id("q4_0", up, E, F, H, ids, T, top_k, x, H, 0, yu)
                bqm.qmv_id("q4_0", down, E, H, F, ids, T, top_k, xd, top_k * F, F, yd)

        ms = time_steps(run, args.steps, args.warmup, torch, not args.no_graph)
        per_expert = 3 * weight_bytes("q4_0", F, H)
        ubytes = sum(L[-1] for L in layers) * per_expert
        abytes = n_layers * 4 * (2 * T * H + 2 * T * top_k * F + T * top_k * F + T * top_k * H)
        gbs = (ubytes + abytes) / (ms * 1e-3) / 1e9
        # per launch: each qmv_id call on its own, bracketed by events on its stream; its
        # algorithmic bytes are the selected experts' matrices plus its inputs and outputs
        launches, lbytes = [], []
        for gate, up, down, ids, x, xd, yg, yu, yd, uniq in layers:
            launches += [lambda w=gate, i=ids, x=x, y=yg: bqm.qmv_id("q4_0", w, E, F, H, i, T, top_k, x, H, 0, y),
                         lambda w=up, i=ids, x=x, y=yu: bqm.qmv_id("q4_0", w, E, F, H, i, T, top_k, x, H, 0, y),
                         lambda w=down, i=ids, x=xd, y=yd: bqm.qmv_id("q4_0", w, E, H, F, i, T, top_k, x, top_k * F, F, y)]
            mat = weight_bytes("q4_0", F, H)
            lbytes += [uniq * mat + 4 * (T * H + T * top_k * F)] * 2       # gate, up
            lbytes += [uniq * mat + 4 * (T * top_k * F + T * top_k * H)]   # down
        dur = per_launch_ms(launches, torch)
        # algorithmic vector work: one FMA per (slot, weight), one code conversion per
        # (selected expert, weight); every expert matrix here has F x H weights
        W = F * H
        n_u = sum(L[-1] for L in layers)
        # from 8 tokens on the indexed products run on the matrix cores (the slot products
        # leave the vector ALU, which keeps one code conversion per weight)
        mma = T >= 8
        fma_id, cvt_id = (0.0 if mma else 3.0 * n_layers * T * top_k * W), 3.0 * n_u * W
        id_kernel = ("k_qmv_id_mma (matrix-core indexed form, Q4_0, groups of up to 16 slots)" if mma else
                     f"k_qmv_chain indexed form (Q4_0, batch class {1 if T == 1 else 2 if T == 2 else 4})")

        # the same layer with gate and up fused (one pass over both, silu(gate) * up out):
        # two launches per layer
        def run_fused():
            for gate, up, down, ids, x, xd, yg, yu, yd, _ in layers:
                bqm.qmv_id_gate_up("q4_0", gate, up, E, F, H, ids, T, top_k, x, H, 0, yg)
                bqm.qmv_id("q4_0", down, E, H, F, ids, T, top_k, xd, top_k * F, F, yd)

        ms_f = time_steps(run_fused, args.steps, args.warmup, torch, not args.no_graph)
        abytes_f = n_layers * 4 * (T * H + T * top_k * F + T * top_k * F + T * top_k * H)
        gbs_f = (ubytes + abytes_f) / (ms_f * 1e-3) / 1e9
        flaunch, fbytes = [], []
        for gate, up, down, ids, x, xd, yg, yu, yd, uniq in layers:
            flaunch.append(lambda g=gate, u=up, i=ids, x=x, y=yg:
                           bqm.qmv_id_gate_up("q4_0", g, u, E, F, H, i, T, top_k, x, H, 0, y))
            fbytes.append(2 * uniq * weight_bytes("q4_0", F, H) + 4 * (T * H + T * top_k * F))
        fdur = per_launch_ms(flaunch, torch)

        # the whole layer fused: gate+up in one pass, then down with the router-weighted
        # sum over each token's experts (its output per token) in one launch
        def run_layer():
            for l, (gate, up, down, ids, x, xd, yg, yu, yd, _) in enumerate(layers):
                bqm.qmv_id_gate_up("q4_0", gate, up, E, F, H, ids, T, top_k, x, H, 0, yg)
                bqm.qmv_id_sum("q4_0", down, E, H, F, ids, rws[l], T, top_k, yg, top_k * F, F, yd,
                               youts[l])

        ms_l = time_steps(run_layer, args.steps, args.warmup, torch, not args.no_graph)
        abytes_l = n_layers * 4 * (T * H + 2 * T * top_k * F + 2 * T * top_k * H + T * H)
        gbs_l = (ubytes + abytes_l) / (ms_l * 1e-3) / 1e9
        slaunch, sbytes = [], []
        for l, (gate, up, down, ids, x, xd, yg, yu, yd, uniq) in enumerate(layers):
            slaunch.append(lambda w=down, i=ids, r=rws[l], x=yg, y=yd, o=youts[l]:
                           bqm.qmv_id_sum("q4_0", w, E, H, F, i, r, T, top_k, x, top_k * F, F, y, o))
            # expert rows, inputs, the weighted slot rows written and read back, the sums
            sbytes.append(uniq * weight_bytes("q4_0", H, F) + 4 * (T * top_k * F + 2 * T * top_k * H + T * H))
        sdur = per_launch_ms(slaunch, torch)
        out.append({"T": T, "ms_per_layer": round(ms / n_layers, 4),
                    "unique_experts_per_layer": [L[-1] for L in layers],
                    "gbs_unique_bytes": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                    "layer_tok_s": round(T * n_layers / (ms * 1e-3), 1),
                    "roofline": binding_roofline(
                        sum(lbytes), fma_id, cvt_id, float(dur.sum()) * 1e-3,
                        id_kernel, round(1e3 * float(dur.mean()), 3), traffic_from_profiles(f"qmv_id_q4_0_moe_t{T}")),
                    "fused_gate_up": {
                        "ms_per_layer": round(ms_f / n_layers, 4), "gbs_unique_bytes": round(gbs_f, 1),
                        "pct_of_hbm_peak": round(100 * gbs_f / HBM_PEAK_GBS, 2),
                        "layer_tok_s": round(T * n_layers / (ms_f * 1e-3), 1),
                        "roofline": binding_roofline(
                            sum(fbytes), (0.0 if mma else 2.0 * n_layers * T * top_k * W), 2.0 * n_u * W,
                            float(fdur.sum()) * 1e-3,
                            ("k_qmv_id_mma gate+up form (qmv_id_gate_up)" if mma else
                             "k_qmv_chain gate+up form (qmv_id_gate_up)"), round(1e3 * float(fdur.mean()), 3),
                            traffic_from_profiles(f"qmv_id_gate_up_q4_0_moe_t{T}"))},
                    "fused_layer": {
                        "what": "qmv_id_gate_up, then qmv_id_sum (down + router-weighted slot sum)",
                        "ms_per_layer": round(ms_l / n_layers, 4), "gbs_unique_bytes": round(gbs_l, 1),
                        "pct_of_hbm_peak": round(100 * gbs_l / HBM_PEAK_GBS, 2),
                        "layer_tok_s": round(T * n_layers / (ms_l * 1e-3), 1),
                        "roofline": binding_roofline(
                            sum(sbytes), (0.0 if mma else 1.0 * n_layers * T * top_k * W), 1.0 * n_u * W,
                            float(sdur.sum()) * 1e-3,
                            ("qmv_id_sum: k_qmv_id_mma (weighted rows) + k_slot_sum" if mma else
                             "qmv_id_sum: k_qmv_chain indexed form (weighted rows) + k_slot_sum"),
                            round(1e3 * float(sdur.mean()), 3), traffic_from_profiles(f"qmv_id_sum_q4_0_moe_t{T}"))}})
        del layers, rws, youts
        torch.cuda.empty_cache()
        if not args.no_cpu:
            say(f"timing the oracle on the host (T = {T}) ...")
            out[-1]["cpu_baseline"] = cpu_baseline_moe(T, E, top_k, H, F, args.cpu_seconds / 2, gen)
    return {"metric": "MoE qmv_id achieved HBM GB/s over unique-expert bytes", "value": out[0]["gbs_unique_bytes"],
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": out[0]["ms_per_layer"] * n_layers, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "128-expert MoE layer (gate/up 4096->1536, down 1536->4096, Q4_0, top-8), "
                                   "8 distinct layers per step"},
            "roofline": out[0]["roofline"],
            **({} if args.no_cpu else {"cpu_baseline": out[0]["cpu_baseline"]}),
            "by_T": out}


def run_prefill(args, torch, gen, bqm, fmt="q8_0"):
    sh = gen.PREFILL_SHAPE
    M, N, K = sh["M"], sh["N"], sh["K"]
    copies = 8
    mats = [make_matrix(fmt, N, K, ("prefill", c), torch, gen, bqm) for c in range(copies)]
    qmm = getattr(bqm, f"qmm_{fmt}")
    X = gen.normal((M, K), ("prefill-x", 0), device="cuda")
    Xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    dx = torch.empty((M, K // 32), device="cuda")
    Y = torch.empty((M, N), device="cuda")
    bqm.bqm_quantize_q8_act(X, Xq, dx, M, K)
    launches = [(lambda w=w: qmm(w, Xq, dx, Y, M, N, K)) for w in mats]
    qlaunch = [lambda: bqm.bqm_quantize_q8_act(X, Xq, dx, M, K)]

    def run():
        bqm.bqm_quantize_q8_act(X, Xq, dx, M, K)
        for f in launches:
            f()

    ms = time_steps(run, args.steps, args.warmup, torch, not args.no_graph)
    dur = per_launch_ms(launches, torch)
    qdur = per_launch_ms(qlaunch, torch)
    ops = 2.0 * M * N * K
    tops = ops / (dur.mean() * 1e-3) / 1e12
    # The binding unit is the vector ALU: every (m, n, block) needs its int32 block sum
    # converted and multiply-added with the scale product (which comes from the matrix
    # cores): 2 lane operations, against 256 CUs x 64 lanes x 2.4 GHz = 39.3 T per second.
    triples = float(M) * N * (K // 32)   # (m, n, block): one conversion and one FMA each
    return {"metric": f"prefill qmm_{fmt} int8 TOP/s", "value": round(tops, 2), "unit": "TOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8/f32",
            "data": "synthetic",
            "config": {"workload": f"prefill GEMM M=512 K=5120 N=17408, {fmt.upper()} weights, 8 weight copies"},
            "roofline": {**alu_roofline(triples, triples, float(dur.mean()) * 1e-3, f"k_qmm_{fmt}",
                                        round(1e3 * float(dur.mean()), 3),
                                        mfma_int8_frac=round(tops / INT8_PEAK_TOPS, 4)),
                         "traffic": traffic_from_profiles(f"qmm_{fmt}_prefill")},
            "quantize_us": round(1e3 * float(qdur.mean()), 3),
            **({} if args.no_cpu else {"cpu_baseline": cpu_baseline_qmm(
                fmt, M, N, K, ("prefill", 0), ("prefill-x", 0), args.cpu_seconds, gen)})}


def run_prefill_moe(args, torch, gen, bqm):
    """The MoE layer over a 512-token prompt: gate and up (4096 -> 1536, one input row per
    token) and down (1536 -> 4096, one input row per slot) through qmm_id, Q4_0 experts."""
    sh = gen.MOE_SHAPE
    E, top_k, H, F, T = sh["E"], sh["top_k"], sh["hidden"], sh["ffn"], gen.MOE_PREFILL_T
    n_layers = 4   # distinct layers (4 x 1.36 GB of experts) cycled
    layers = []
    for l in range(n_layers):
        gate = make_matrix("q4_0", E * F, H, ("moep", l, "gate"), torch, gen, bqm)
        up = make_matrix("q4_0", E * F, H, ("moep", l, "up"), torch, gen, bqm)
        down = make_matrix("q4_0", E * H, F, ("moep", l, "down"), torch, gen, bqm)
        ids_np = gen.router_ids(T, E, top_k, ("moep-ids", l))
        ids = torch.from_numpy(ids_np).cuda()
        x = gen.normal((T, H), ("moep-x", l), device="cuda")
        xq = torch.empty((T, H), dtype=torch.int8, device="cuda")
        xdx = torch.empty((T, H // 32), device="cuda")
        bqm.bqm_quantize_q8_act(x, xq, xdx, T, H)
        h = gen.normal((T * top_k, F), ("moep-h", l), device="cuda")
        hq = torch.empty((T * top_k, F), dtype=torch.int8, device="cuda")
        hdx = torch.empty((T * top_k, F // 32), device="cuda")
        bqm.bqm_quantize_q8_act(h, hq, hdx, T * top_k, F)
        yg = torch.empty((T, top_k, F), device="cuda")
        yu = torch.empty((T, top_k, F), device="cuda")
        yd = torch.empty((T, top_k, H), device="cuda")
        counts = np.bincount(ids_np.ravel(), minlength=E)
        layers.append((gate, up, down, ids, xq, xdx, hq, hdx, yg, yu, yd, counts))

    def run():
        for gate, up, down, ids, xq, xdx, hq, hdx, yg, yu, yd, _ in layers:
            bqm.qmm_id("q4_0", gate, E, F, H, ids, T, top_k, xq, xdx, 1, 0, yg)
            bqm.qmm_id("q4_0", up, E, F, H, ids, T, top_k, xq, xdx, 1, 0, yu)
            bqm.qmm_id("q4_0", down, E, H, F, ids, T, top_k, hq, hdx, top_k, 1, yd)

    ms = time_steps(run, args.steps, args.warmup, torch, not args.no_graph)
    launches = []
    for gate, up, down, ids, xq, xdx, hq, hdx, yg, yu, yd, _ in layers:
        launches += [lambda w=gate, i=ids, a=xq, d=xdx, y=yg: bqm.qmm_id("q4_0", w, E, F, H, i, T, top_k, a, d, 1, 0, y),
                     lambda w=up, i=ids, a=xq, d=xdx, y=yu: bqm.qmm_id("q4_0", w, E, F, H, i, T, top_k, a, d, 1, 0, y),
                     lambda w=down, i=ids, a=hq, d=hdx, y=yd: bqm.qmm_id("q4_0", w, E, H, F, i, T, top_k, a, d, top_k, 1, y)]
    dur = per_launch_ms(launches, torch)
    slots = T * top_k
    ops = n_layers * 3 * 2.0 * slots * F * H           # useful int8 operations, all launches
    tops = ops / (dur.sum() * 1e-3) / 1e12
    triples = n_layers * 3.0 * slots * F * (H // 32)  # (slot, n, block): one conversion, one FMA
    # algorithmic HBM bytes of all launches: each selected expert's weights once, the int8
    # inputs and their block scales once, the outputs written
    hbm_bytes = 0
    for L in layers:
        U = int(np.sum(L[-1] > 0))
        hbm_bytes += 2 * (U * F * (H // 32) * 18 + T * H + T * (H // 32) * 4 + slots * F * 4)  # gate, up
        hbm_bytes += U * H * (F // 32) * 18 + slots * F + slots * (F // 32) * 4 + slots * H * 4  # down
    # the kernel's row tiles: 64 slots of an expert while more than 32 are left, then 32
    tall = [int(np.sum(L[-1] // 64 + (L[-1] % 64 > 32))) for L in layers]
    short = [int(np.sum((L[-1] % 64 > 0) & (L[-1] % 64 <= 32))) for L in layers]
    return {"metric": "MoE prefill qmm_id int8 TOP/s", "value": round(tops, 2), "unit": "TOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8/f32",
            "data": "synthetic",
            "config": {"workload": "128-expert MoE layer (gate/up 4096->1536, down 1536->4096, Q4_0, top-8) "
                                   "over a 512-token prompt, 4 distinct layers per step"},
            "ms_per_layer": round(ms / n_layers, 4),
            "busiest_expert_slots": [int(L[-1].max()) for L in layers],
            "row_tile_fill": round(slots / float(np.mean([64 * a + 32 * b for a, b in zip(tall, short)])), 3),
            # the binding roofline: each selected expert's weights cross HBM once (with
            # half the experts holding two slots or fewer, the weights take longer at 8 TB/s
            # than the useful products' vector work takes at its rates), or the vector ALU
            "roofline": {**binding_roofline(hbm_bytes, triples, triples, float(dur.sum()) * 1e-3,
                                            "k_qmm_id_q4_0", round(1e3 * float(dur.mean()), 3),
                                            traffic_from_profiles("qmm_id_q4_0_moe_prefill")),
                         "mfma_int8_frac": round(tops / INT8_PEAK_TOPS, 4)},
            **({} if args.no_cpu else {"cpu_baseline": cpu_baseline_qmm_id(
                E, top_k, H, F, T, args.cpu_seconds, gen)})}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU sharding "
              f"is a design note, not built", file=sys.stderr)
        sys.exit(2)
    import torch
    import gen
    from block_quantized_matrix_amd import bqm
    bqm.lib()   # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    say(f"device: {torch.cuda.get_device_name(0)}")
    wl = args.workload
    if wl == "dense27b_q4_0":
        res = run_dense(args, torch, gen, bqm, "q4_0")
    elif wl == "dense27b_q8_0":
        res = run_dense(args, torch, gen, bqm, "q8_0")
    elif wl == "gemv4096":
        res = run_gemv4096(args, torch, gen, bqm)
    elif wl == "moe":
        res = run_moe(args, torch, gen, bqm)
    elif wl == "prefill_q4_0":
        res = run_prefill(args, torch, gen, bqm, "q4_0")
    elif wl == "prefill_moe":
        res = run_prefill_moe(args, torch, gen, bqm)
    else:
        res = run_prefill(args, torch, gen, bqm)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

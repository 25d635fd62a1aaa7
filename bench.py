"""Benchmark of the ring-decomposed AG+GEMM (and GEMM+RS) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ag_4k|ag_qkv|ag_fc1_f8|rs_8k]

A step is one ag_gemm call (or one gemm_rs call for rs_8k) through the C ABI on inputs already
resident in HBM: with the default engine, one GEMM launch whose waiting workgroups copy the peers'
chunks into G and release their counters.  The default workload is AG+GEMM at M=K=N=4096, tp=4,
self_rank=1, bf16.  The default warm-up (1000 steps) lets the chip's clock settle before the
timed steps; the timed steps are bracketed by one event pair, and the per-step and per-kernel
figures come from a separate instrumented pass right after them.

Prints one JSON line: throughput (TFLOP/s) of the whole step, the overlap figures (chunked,
GEMM-only and copy-only times of the same kernels measured back to back after the headline, overlap
ratio T_chunked / (T_copy_only + T_gemm_only), the hidden fraction of the copy time, the headline's
time over that chunked time, and the same work without overlap in one step: the copies-only
launch followed by the GEMM-only launch), the roofline of the GEMM kernel (algorithmic flops per
launch over its average launch duration, from HIP events that each launch records on the stream
it runs on), for AG a timeline of one traced call (chunk releases against tile starts; the stamps
slow a traced call by some 15%, so its times are relative) and the CPU oracle's throughput on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2}   # 256 CU x 2.4 GHz x (4096 | 8192) flop/clk

PEAK_HBM_GBS = 8000.0
METRICS = {
    "ag": "AG+GEMM TFLOP/s (+% MFMA peak) and overlap efficiency, M=K=N=4096 tp=4",
    "rs": "GEMM+RS TFLOP/s (+% MFMA peak) and epilogue HBM GB/s",
}


def set_engine(ctx, B, name):
    """Copy engine by name; "in-gemm-slab" is the in-GEMM engine with K-slab gating (AG+GEMM; a
    GEMM+RS call treats it as the in-GEMM engine)."""
    ctx.set_option(B.RAG_OPT_COPY_ENGINE, B.ENGINES[name.replace("-slab", "")])
    ctx.set_option(B.RAG_OPT_AG_GATE,
                   B.RAG_GATE_SLAB if name.endswith("-slab") else B.RAG_GATE_CHUNK)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # The chip's clock settles only after some 25 ms of sustained calls (from idle, the first 50
    # ag_4k calls run 16% slower than the steady state); the default warm-up covers that.
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=1000)
    p.add_argument("--workload", default="ag_4k")
    p.add_argument("--copy-engine", default=os.environ.get("RAG_COPY_ENGINE", "in-gemm"),
                   choices=["kernel", "sdma", "in-gemm", "in-gemm-slab", "assist", "in-gemm-sdma"])
    p.add_argument("--comm-cus", type=int, default=0,
                   help="compute units the side stream's copy kernels are limited to (0 = all)")
    p.add_argument("--sdma-streams", type=int, default=1,
                   help="side streams the SDMA engine spreads its copies over (1-3)")
    p.add_argument("--own-chunk", default="in-g", choices=["in-g", "separate"],
                   help="in-g: the own chunk lives in its slot of G, as the local shard does in a "
                        "ring all-gather; separate: it is its own buffer and is copied into G")
    p.add_argument("--comm-wgs", type=int, default=int(os.environ.get("RAG_COMM_WGS", "128")),
                   help="workgroups of the side-stream copy kernel (side-stream engine and the "
                        "split form)")
    p.add_argument("--tile", default=os.environ.get("RAG_TILE", "auto"))
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target wall time of the CPU oracle sample")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--no-timeline", action="store_true",
                   help="AG: skip the timeline (after the timed steps, 20 more calls traced with "
                        "the library's per-tile wall-clock stamps: for the last, when each chunk "
                        "was released and when its tiles ran)")
    p.add_argument("--flush-calls", type=int, default=50,
                   help="RS: calls timed with the MALL scrubbed before each (a 512 MiB write)")
    p.add_argument("--headline-only", action="store_true",
                   help="measure the headline call (and, for AG, its GEMM-only and copies-only "
                        "forms) but none of the other variants; for counter-collection runs, "
                        "where the profiler serialises dispatches and a GEMM whose arrivals come "
                        "from a kernel on another stream would wait for it in vain")
    return p.parse_args()


_CHECK = None   # the context's check (raises if a counter wait timed out), set in main()


def progress(msg: str):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def time_steps(fn, steps, warmup, stream, label="step"):
    """Average ms per step over `steps` back-to-back steps after `warmup` untimed ones, bracketed
    by one event pair (and a synchronisation on both sides): nothing else is enqueued between the
    steps.  The first warm-up step is checked on its own, so that a call whose waits time out
    fails the benchmark at once instead of after every step has waited out its limit."""
    import torch
    w0 = time.perf_counter()
    if warmup > 0:
        fn()
        torch.cuda.synchronize()
        if _CHECK is not None:
            _CHECK()
    for _ in range(warmup - 1):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    progress(f"{label}: {ms:.5f} ms per step ({time.perf_counter() - w0:.1f} s)")
    return ms


def per_step_times(fn, steps, stream):
    """ms of each of `steps` steps, from an event pair around each (a separate, instrumented pass:
    each event record costs a few microseconds of queue time)."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        stops[i].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in zip(starts, stops)]


def rnd(x, nd=5):
    return None if x is None else round(x, nd)


def pctl(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


def cpu_baseline_ag(inp, target_s, D_timed):
    """The oracle (as it stands) on whole output rows of the same workload; sample sized so the
    timed part takes about target_s seconds of wall time (all rows when they fit).  The rows it
    computes are also the reference for the output of the last timed GPU step: returns
    (baseline, parity)."""
    import numpy as np
    from oracle import ringag_oracle as O
    from ring_all_gather_amd import workloads as W
    s = inp.shape
    fp8 = s.dtype == "fp8"
    conv = (lambda t: O.dequantize_e4m3(W.bits_u8(t), inp.scale_B)) if fp8 else \
        (lambda t: O.bf16_to_f32(W.bits_u16(t)))
    A = O.dequantize_e4m3(W.bits_u8(inp.A), inp.scale_A) if fp8 else O.bf16_to_f32(
        W.bits_u16(inp.A))
    G = O.gather([conv(c) for c in inp.chunks])
    flops_row = 2.0 * s.M * s.K
    probe = np.arange(0, min(s.N, 16))
    t = time.perf_counter()
    O.gemm_tn_rows(G, A, probe)
    dt = max(time.perf_counter() - t, 1e-4)
    nrows = int(min(s.N, max(16, len(probe) * target_s / dt)))
    rows = np.linspace(0, s.N - 1, nrows).astype(np.int64)
    t = time.perf_counter()
    ref = O.gemm_tn_rows(G, A, rows)
    dt = time.perf_counter() - t
    base = {"value": round(flops_row * nrows / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": O.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{nrows} of the {s.N} output rows (each {s.M}x{s.K} MACs, fp32 triple loop "
                      f"over the gathered input), {dt:.1f} s wall"}
    got = O.bf16_to_f32(W.bits_u16(D_timed.cpu()))[rows].astype(np.float64)
    err = float(np.abs(got - ref).max() / max(float(np.abs(ref).max()), 1e-30))
    tol = 5e-2 if fp8 else 2e-2
    par = {"rows_checked": int(nrows), "of_rows": int(s.N), "max_rel_err": round(err, 6),
           "tolerance": tol, "ok": bool(np.isfinite(err) and err <= tol)}
    return base, par


def cpu_baseline_rs(inp, target_s, D_timed, send_timed):
    """The oracle on whole rows of the local partial X W^T (sample sized for about target_s
    seconds, all rows when they fit).  Those rows are also the reference for the outgoing chunks
    of the last timed GPU step (send[c] = rows of chunk c of the partial), and the oracle's
    reduce-scatter on the own chunk's sampled rows is the reference for its D: returns (baseline,
    parity)."""
    import numpy as np
    from oracle import ringag_oracle as O
    from ring_all_gather_amd import workloads as W
    s = inp.shape
    Xb, Wb = W.bits_u16(inp.X), W.bits_u16(inp.W)
    Xf, Wf = O.bf16_to_f32(Xb), O.bf16_to_f32(Wb)
    flops_row = 2.0 * s.Mo * s.Kl
    probe = np.arange(0, 16)
    t = time.perf_counter()
    O.gemm_tn_rows(Xf, Wf, probe)
    dt = max(time.perf_counter() - t, 1e-4)
    nrows = int(min(s.T, max(16, len(probe) * target_s / dt)))
    rows = np.linspace(0, s.T - 1, nrows).astype(np.int64)
    t = time.perf_counter()
    P_rows = O.gemm_tn_rows(Xf, Wf, rows)
    dt = time.perf_counter() - t
    base = {"value": round(flops_row * nrows / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": O.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{nrows} of the {s.T} rows of the local partial X W^T (each {s.Mo}x{s.Kl} "
                      f"MACs, fp32 triple loop), {dt:.1f} s wall"}
    send = send_timed.cpu().numpy()
    chunk = rows // s.nc
    out_rows = chunk != s.self_rank
    got_send = send[chunk[out_rows], rows[out_rows] % s.nc]
    ref_send = P_rows[out_rows]
    e_send = float(np.abs(got_send - ref_send).max() / max(float(np.abs(ref_send).max()), 1e-30))
    own = rows[~out_rows] - s.self_rank * s.nc
    peers = [None if p is None else p.numpy() for p in inp.partials]
    D_ref = O.gemm_rs_rows(Xb, Wb, peers, s.tp, s.self_rank, own)
    got_D = O.bf16_to_f32(W.bits_u16(D_timed.cpu()))[own].astype(np.float64)
    e_D = float(np.abs(got_D - D_ref).max() / max(float(np.abs(D_ref).max()), 1e-30))
    par = {"rows_checked": int(nrows), "of_rows": int(s.T), "D_rows_checked": int(len(own)),
           "max_rel_err_D": round(e_D, 6), "max_rel_err_send": round(e_send, 8),
           "tolerance_D": 2e-2, "tolerance_send": 1e-3,
           "ok": bool(e_D <= 2e-2 and e_send <= 1e-3)}
    return base, par


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the CPU baseline."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def timeline_ag(ctx, B, step, shape, kname):
    """The last of 20 back-to-back traced calls (RAG_OPT_TRACE_BUF: every traced call overwrites
    the stamps; 100 MHz wall clock): per ring position, when the chunk was released and when the
    first of its tiles started computing and the last ended, in microseconds from the first
    tile's start.  The stamps themselves slow a traced call (by some 15% at ag_4k)."""
    import math
    import re
    import torch
    m = re.search(r"_t(\d+)x(\d+)", kname)
    bi, bj = int(m.group(1)), int(m.group(2))
    per_chunk = math.ceil(shape.nc / bi) * math.ceil(shape.M / bj)
    total = per_chunk * shape.tp
    buf = torch.zeros(64 + 5 * total, dtype=torch.int64, device="cuda:0")
    ctx.set_trace(buf)
    for _ in range(20):
        step()
    ctx.set_trace(None)
    torch.cuda.synchronize()
    w = buf.cpu().tolist()
    tiles = [w[64 + 5 * t: 64 + 5 * t + 5] for t in range(total)]
    t0 = min(x[0] for x in tiles)
    us = lambda v: round((v - t0) / 100.0, 2)
    chunks = []
    for j in range(shape.tp):
        tj = tiles[j * per_chunk:(j + 1) * per_chunk]
        chunks.append({"ring_pos": j, "rank": (shape.self_rank - j) % shape.tp,
                       # (K-slab gating releases slabs, not chunks: no chunk stamp)
                       "released_us": 0.0 if j == 0 else (us(w[j - 1]) if w[j - 1] else None),
                       "first_tile_go_us": us(min(x[1] for x in tj)),
                       "last_tile_end_us": us(max(x[2] for x in tj))})
    # the core clock the tiles ran at: s_memtime cycles over the 100 MHz wall time of each tile's
    # computation (from after its wait to its end), in GHz
    clk = sorted(x[4] / ((x[2] - x[1]) * 10.0) for x in tiles if x[2] > x[1])
    q = lambda f: round(clk[min(len(clk) - 1, int(f * len(clk)))], 3) if clk else None
    return {"tiles_per_chunk": per_chunk, "copies_start_us": us(w[32]),
            "gemm_end_us": us(max(x[2] for x in tiles)),
            "tile_clock_ghz": {"p10": q(0.1), "p50": q(0.5), "p90": q(0.9)}, "chunks": chunks}


def overlap_per_engine(ctx, B, step, args, stream, shape):
    """T_gemm_only, T_copy_only, T_chunked, the overlap ratio and the hidden fraction for the
    headline copy engine and, unless --headline-only, for the other engines.  An engine's three
    times are measured back to back (its chunked call again for the headline engine), so that
    they come from one regime of the clock: with a short warm-up the headline's own steps still
    run while the clock ramps up from idle, and setting them against legs timed later would
    charge the ramp to the overlap.  Each engine's GEMM-only launch uses the tile its chunked
    call uses (the side-stream kernel engine may pick another kernel of the same tile size, see
    the library's tile choice), so the three times are of the same kernel."""
    names = [args.copy_engine] + ([] if args.headline_only else
                                  [e for e in ("in-gemm", "in-gemm-slab", "assist", "in-gemm-sdma",
                                               "kernel", "sdma") if e != args.copy_engine])
    res = {}
    for eng in names:
        set_engine(ctx, B, eng)
        kname = ctx.ag_kernel_name(shape.nc, shape.M, shape.tp, shape.dtype == "fp8")
        t_chunked = time_steps(step, args.steps, args.warmup, stream, f"{eng} chunked")
        t_copy = time_steps(lambda: step(B.RAG_COPY_ONLY), args.steps, args.warmup, stream,
                            f"{eng} copies only")
        tile = kname.split("_t", 1)[1]
        if args.tile == "auto":
            ctx.set_option(B.RAG_OPT_TILE, B.TILES[tile])
        t_gemm = time_steps(lambda: step(B.RAG_NO_COPY), args.steps, args.warmup, stream,
                            f"{eng} GEMM only")
        ctx.set_option(B.RAG_OPT_TILE, B.TILES[args.tile])
        ctx.check()
        res[eng] = {"kernel": kname, "t_chunked_ms": round(t_chunked, 5),
                    "t_gemm_only_ms": round(t_gemm, 5), "t_copy_only_ms": round(t_copy, 5),
                    "overlap_ratio": round(t_chunked / (t_copy + t_gemm), 4),
                    "hidden_fraction": round((t_copy + t_gemm - t_chunked) / t_copy, 4)}
    return res


def measured_traffic(workload: str, kernel: str, fingerprint: str):
    """HBM bytes per launch from the committed counter record of this workload, if it was taken
    with this exact build of the kernels and this kernel; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{workload}_gemm_hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernels_sha256") != fingerprint or rec.get("kernel") != kernel:
        return None
    return rec.get("traffic_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs one rank's share on one GPU; --gpus {args.gpus} is not supported "
              "(the ring's peers are simulated on the same device)", file=sys.stderr)
        return 2
    import torch
    from ring_all_gather_amd import binding as B
    from ring_all_gather_amd import workloads as W

    dev = "cuda:0"
    # every call goes on a stream of the bench's own: a side stream limited to some compute units
    # is blocking with respect to the null stream, which would serialise its copies with the GEMM
    torch.cuda.set_stream(torch.cuda.Stream())
    ctx = B.Context(0, max_tp=16)
    global _CHECK
    _CHECK = ctx.check
    set_engine(ctx, B, args.copy_engine)
    ctx.set_option(B.RAG_OPT_COMM_WGS, args.comm_wgs)
    ctx.set_option(B.RAG_OPT_TILE, B.TILES[args.tile])
    ctx.set_option(B.RAG_OPT_COMM_CUS, args.comm_cus)
    ctx.set_option(B.RAG_OPT_SDMA_STREAMS, args.sdma_streams)
    shape = W.WORKLOADS[args.workload]
    stream = torch.cuda.current_stream()
    out = {}

    if isinstance(shape, W.AGShape):
        inp = W.make_ag(shape)
        A = inp.A.to(dev)
        G = torch.empty((shape.N, shape.K), dtype=inp.A.dtype, device=dev)
        chunks = [c.to(dev) for c in inp.chunks]
        if args.own_chunk == "in-g":
            s0 = shape.self_rank * shape.nc
            G[s0:s0 + shape.nc].copy_(chunks[shape.self_rank])
            chunks[shape.self_rank] = G[s0:s0 + shape.nc]
        D = torch.empty((shape.N, shape.M), dtype=torch.bfloat16, device=dev)
        sA = sB = None
        if shape.dtype == "fp8":
            sA = torch.tensor([inp.scale_A], dtype=torch.float32, device=dev)
            sB = torch.tensor([inp.scale_B], dtype=torch.float32, device=dev)

        def step(flags=0):
            B.ag_gemm(ctx, A, chunks, shape.tp, shape.self_rank, D, G=G, scale_A=sA, scale_B=sB,
                      flags=flags)

        ms = time_steps(step, args.steps, args.warmup, stream, "chunked (headline)")
        D_timed = D.clone()   # the output of the last timed step, checked against the oracle
        # instrumented pass right after it: per-step events, and the library's events around each
        # GEMM launch on the stream it runs on (the roofline's kernel duration)
        ctx.kernel_times()
        ctx.set_option(B.RAG_OPT_TIMING, 1)
        per = per_step_times(step, args.steps, stream)
        kt = ctx.kernel_times()
        ctx.set_option(B.RAG_OPT_TIMING, 0)
        ctx.check()
        kname = ctx.ag_kernel_name(shape.nc, shape.M, shape.tp, shape.dtype == "fp8")
        engines = overlap_per_engine(ctx, B, step, args, stream, shape)
        head = engines[args.copy_engine]
        ms_pair = head["t_chunked_ms"]
        ms_gemm, ms_copy = head["t_gemm_only_ms"], head["t_copy_only_ms"]
        ms_staged = ms_split = ms_seq = None
        if not args.headline_only:
            set_engine(ctx, B, args.copy_engine)
            ms_staged = time_steps(lambda: step(B.RAG_STAGED_OUT), args.steps, args.warmup,
                                   stream, "staged output")
            # the split form (one GEMM launch per chunk, gated by stream events): what the
            # in-kernel counters buy
            ms_split = time_steps(lambda: step(B.RAG_PER_CHUNK), args.steps, args.warmup, stream,
                                  "split form")
            # the same work without overlap: the copies-only launch, then the GEMM-only launch
            ms_seq = time_steps(lambda: (step(B.RAG_COPY_ONLY), step(B.RAG_NO_COPY)), args.steps,
                                args.warmup, stream, "copies then GEMM")
        ctx.check()
        set_engine(ctx, B, args.copy_engine)
        flops = shape.flops
        kernel_ms = statistics.fmean(kt)
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        traffic = measured_traffic(args.workload, kname, B.kernels_fingerprint())
        peak = PEAK_TFLOPS[shape.dtype]
        value = flops / (ms * 1e-3) / 1e12
        out = {
            "metric": METRICS["ag"] if args.workload == "ag_4k" else
            f"AG+GEMM TFLOP/s (+% MFMA peak) and overlap efficiency, {args.workload}",
            "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": shape.dtype, "data": "synthetic",
            "config": {"workload": f"ag_gemm tp={shape.tp} self_rank={shape.self_rank} "
                                   f"N={shape.N} (chunks of {shape.nc}) M={shape.M} K={shape.K} "
                                   f"{shape.dtype}",
                       "tp": shape.tp, "self_rank": shape.self_rank, "N": shape.N, "M": shape.M,
                       "K": shape.K, "copy_engine": args.copy_engine, "own_chunk": args.own_chunk,
                       "comm_wgs": args.comm_wgs, "comm_cus": args.comm_cus,
                       "sdma_streams": args.sdma_streams, "tile": args.tile},
            "pct_mfma_peak": round(100.0 * value / peak, 2),
            "step_ms": {"p10": round(pctl(per, 0.1), 5), "p50": round(pctl(per, 0.5), 5),
                        "p90": round(pctl(per, 0.9), 5)},
            "overlap": {"t_chunked_ms": round(ms_pair, 5), "t_gemm_only_ms": round(ms_gemm, 5),
                        "t_copy_only_ms": round(ms_copy, 5),
                        "overlap_ratio": round(ms_pair / (ms_copy + ms_gemm), 4),
                        "hidden_fraction": round((ms_copy + ms_gemm - ms_pair) / ms_copy, 4),
                        "headline_vs_chunked_pair": round(ms / ms_pair, 4),
                        "t_copy_then_gemm_ms": rnd(ms_seq),
                        "chunked_vs_copy_then_gemm": rnd(ms_seq and ms_pair / ms_seq, 4),
                        "t_staged_out_ms": rnd(ms_staged),
                        "t_split_per_chunk_ms": rnd(ms_split),
                        "per_engine": engines},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                         "kernel": kname, "kernel_ms": round(kernel_ms, 5)},
        }
        if not args.no_timeline:
            out["timeline"] = timeline_ag(ctx, B, step, shape, kname)
        # the gathered buffer must hold every chunk at its rank offset, bit for bit
        G_ok = all(torch.equal(G[r * shape.nc:(r + 1) * shape.nc].view(torch.uint8),
                               chunks[r].view(torch.uint8)) for r in range(shape.tp))
        out["parity"] = {"G_equals_chunks": bool(G_ok)}
        if not args.no_cpu:
            base, par = cpu_baseline_ag(inp, args.cpu_seconds, D_timed)
            out["cpu_baseline"] = base
            out["parity"].update(par)
    else:
        inp = W.make_rs(shape)
        X, Wt = inp.X.to(dev), inp.W.to(dev)
        parts = [None if p is None else p.to(dev) for p in inp.partials]
        D = torch.empty((shape.nc, shape.Mo), dtype=torch.bfloat16, device=dev)
        send = torch.empty((shape.tp, shape.nc, shape.Mo), dtype=torch.float32, device=dev)

        def step():
            B.gemm_rs(ctx, X, Wt, parts, shape.tp, shape.self_rank, D, send=send)

        ms = time_steps(step, args.steps, args.warmup, stream, "gemm_rs (headline)")
        D_timed, send_timed = D.clone(), send.clone()   # checked against the oracle below
        ctx.kernel_times()
        ctx.set_option(B.RAG_OPT_TIMING, 1)
        per = per_step_times(step, args.steps, stream)
        kt = ctx.kernel_times()
        ctx.set_option(B.RAG_OPT_TIMING, 0)
        kernel_ms = statistics.fmean(kt)
        flops = shape.flops
        nc, Mo, tp = shape.nc, shape.Mo, shape.tp
        kname = ctx.rs_kernel_name(nc, Mo, tp)
        alg_bytes = (shape.T * shape.Kl * 2 + Mo * shape.Kl * 2 + (tp - 1) * nc * Mo * 4 * 2
                     + nc * Mo * 2)
        value = flops / (ms * 1e-3) / 1e12
        gbs = alg_bytes / (kernel_ms * 1e-3) / 1e9
        out = {
            "metric": METRICS["rs"], "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"gemm_rs tp={tp} self_rank={shape.self_rank} T={shape.T} "
                                   f"Kl={shape.Kl} Mo={Mo} bf16, fp32 partials and send",
                       "tile": args.tile},
            "pct_mfma_peak": round(100.0 * value / PEAK_TFLOPS["bf16"], 2),
            "step_ms": {"p10": round(pctl(per, 0.1), 5), "p50": round(pctl(per, 0.5), 5),
                        "p90": round(pctl(per, 0.9), 5)},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic(args.workload, kname,
                                                     B.kernels_fingerprint()),
                         "kernel": kname, "kernel_ms": round(kernel_ms, 5),
                         "algorithmic_bytes": alg_bytes},
        }
        if not args.headline_only:
            # the same launch with the 256 MB MALL scrubbed before each call (a 512 MiB buffer
            # written in between), timed by the launches' own events: the partials and operands
            # then come from HBM, not from the memory-side cache that holds them in steady state
            scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
            ctx.kernel_times()
            ctx.set_option(B.RAG_OPT_TIMING, 1)
            for i in range(args.flush_calls):
                scrub.fill_(i & 0xFF)
                step()
            torch.cuda.synchronize()
            kt_flushed = ctx.kernel_times()
            ctx.set_option(B.RAG_OPT_TIMING, 0)
            del scrub
            kms_f = statistics.fmean(kt_flushed)
            gbs_f = alg_bytes / (kms_f * 1e-3) / 1e9
            out["mall_scrubbed"] = {"calls": len(kt_flushed), "kernel_ms": round(kms_f, 5),
                                    "achieved_GBps": round(gbs_f, 1),
                                    "frac": round(gbs_f / PEAK_HBM_GBS, 4),
                                    "tflops": round(flops / (kms_f * 1e-3) / 1e12, 2)}
            # the counter-gated forms: the peers' partials arrive during the call (copies in ring
            # order, run by the GEMM's own workgroups with the in-GEMM engine, else beside it;
            # tiles wait before their epilogue), and one ring-accumulate step with its incoming
            # running sums given or arriving
            ms_arrive = time_steps(
                lambda: B.gemm_rs(ctx, X, Wt, parts, shape.tp, shape.self_rank, D, send=send,
                                  flags=B.RAG_RS_ARRIVE), args.steps, args.warmup, stream,
                "gemm_rs, partials arrive")
            rin = W.make_rs_ring(shape)
            inc = [t.to(dev) for t in rin.incoming]
            Xr, Wr = rin.X.to(dev), rin.W.to(dev)
            ms_ring = time_steps(
                lambda: B.gemm_rs_ring(ctx, Xr, Wr, inc, shape.tp, shape.self_rank, D, send=send),
                args.steps, args.warmup, stream, "ring step, sums given")
            ms_ring_arrive = time_steps(
                lambda: B.gemm_rs_ring(ctx, Xr, Wr, inc, shape.tp, shape.self_rank, D, send=send,
                                       flags=B.RAG_RS_ARRIVE), args.steps, args.warmup, stream,
                "ring step, sums arrive")
            # the row-parallel linear with its output all-reduced: the reduce-scatter above plus
            # an all-gather of the owners' reduced chunks into Y, copied beside the GEMM
            red = [t.to(dev) for t in W.make_reduced_chunks(shape)]
            Y = torch.empty((shape.T, shape.Mo), dtype=torch.bfloat16, device=dev)
            ms_lar = time_steps(
                lambda: B.linear_allreduce(ctx, X, Wt, parts, red, shape.tp, shape.self_rank, Y,
                                           send=send), args.steps, args.warmup, stream,
                "linear_allreduce")
            ctx.check()
            # the gathered chunks of Y after the timed steps: bit for bit the owners' reduced chunks
            nc_ = shape.nc
            y_gather_ok = all(
                torch.equal(Y[c * nc_:(c + 1) * nc_].view(torch.int16), red[c].view(torch.int16))
                for c in range(shape.tp) if c != shape.self_rank)
            out["variants_ms_per_step"] = {
                "one_shot_partials_given": round(ms, 5),
                "one_shot_partials_arrive": round(ms_arrive, 5),
                "ring_step_sums_given": round(ms_ring, 5),
                "ring_step_sums_arrive": round(ms_ring_arrive, 5),
                "linear_allreduce": round(ms_lar, 5),
                "linear_allreduce_gather_bitwise_ok": bool(y_gather_ok),
                "arrival_engine": args.copy_engine,
                "comm_wgs": args.comm_wgs}
        if not args.no_cpu:
            out["cpu_baseline"], out["parity"] = cpu_baseline_rs(inp, args.cpu_seconds, D_timed,
                                                                 send_timed)
    ctx.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

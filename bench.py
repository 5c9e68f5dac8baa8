#!/usr/bin/env python3
"""Benchmark of the fused-dequant quantized GEMV path on one MI355X.

Workload (the headline configuration): Q4_0 weights at the dense FFN gate
shape N=21504, K=5376, M=1 -- one plain matrix-vector product and one gated
GELU pair over two independent matrices of that shape.  One step = both
products over one activation vector.  Inputs are seeded synthetic data with
the weight/activation distributions of the block formats; they are resident
in HBM before timing starts.  Four independent slot sets (781 MB, more than
twice the 256 MB last-level cache) are rotated so that every step streams its
weights from HBM, as a decoder streams each layer's weights once per token.

Metric: effective GB/s = algorithmic bytes (weights + activations + outputs)
per step / time per step, and the fraction of the 8 TB/s HBM peak.

Timing: the K timed steps are split into --reps windows (3 by default) with
events between them; `value` and `ms_per_step` are the median window, and
the windows' spread is reported.  Per-kernel durations are the median of
--reps repetitions of a back-to-back loop of each entry point alone, rotating
over all twelve matrices of the slot sets (780 MB).

Usage: python bench.py [--gpus 1] [--steps 300] [--warmup 20] [--reps 3] [--no-rows] [--no-cpu-baseline]
Prints one JSON line.  `--trace-summary DIR` / `--pmc-summary DIR` instead
print the markdown summaries kept under profiles/ from rocprofv3 CSV output.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
PREWARM_MS = 50.0  # untimed load before the timed loops (see main)
INT8_MFMA_PEAK_TOPS = 5000.0  # MI355X published dense int8 MFMA rate
ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# HBM traffic per launch comes from the committed rocprofv3 counter summary
# (FETCH_SIZE / WRITE_SIZE, scaled by a plain copy); it is reported only while
# the sources it was measured on are unchanged.
TRAFFIC_PROFILE = os.path.join("profiles", "qmv_bench_workloads_counters.md")
# kernel symbol of each timed launch, and its workgroups per CU at most
KERNEL_OF = {
    "qmv_q4_0": ("qmv::gemv_unit_kernel<0, 1, false, false>", 3),
    "qmv_q4_0_geglu": ("qmv::gemv_unit_kernel<0, 1, true, false>", 8),
}


def unit_grid(N: int, K: int, cus: int, per_cu: int) -> int:
    """Workgroups of the unit GEMV launch: 4 waves per workgroup, one pass of
    64 // (K/256) rows per wave, capped at per_cu workgroups per CU."""
    rows_per_pass = 64 // (K // 256)
    npasses = -(-N // rows_per_pass)
    return min(-(-npasses // 4), cus * per_cu)


def profiled_traffic(kernel: str, grid: int):
    """HBM bytes (read + write) per launch of `kernel` from the counter
    summary, or None when it is missing or was taken on other sources."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    try:
        text = open(path).read()
    except OSError:
        return None
    if not _sources_match(text):
        return None
    for name, g, rd, wr in re.findall(r"<!-- traffic (.+?) grid=(\d+) read=(\d+) write=(\d+) -->", text):
        if name == kernel and int(g) == grid:
            return int(rd) + int(wr)
    return None


# Kernel-trace means of the two timed launches come from a trace of the
# headline loops alone (bench.py --no-rows): in the full run other rows launch
# the same kernels at the same grid on other data (e.g. eight rows over one
# matrix), which would mix into the mean.
TRACE_PROFILE = os.path.join("profiles", "qmv_bench_headline_kernel_trace.md")


def _sources_match(text):
    """True when every `source_sha256 <file> <digest>` line of a profile
    summary matches the file as it is now."""
    import hashlib
    pairs = re.findall(r"source_sha256 (\S+) ([0-9a-f]{64})", text)
    if not pairs:
        return False
    for src, digest in pairs:
        try:
            with open(os.path.join(ROOT, src), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest:
                    return False
        except OSError:
            return False
    return True


def profiled_trace_us(kernel: str, grid: int):
    """Mean kernel-trace duration (us) of `kernel` at `grid` workgroups from the
    committed trace summary, or None when it is missing or was taken on other
    sources."""
    try:
        text = open(os.path.join(ROOT, TRACE_PROFILE)).read()
    except OSError:
        return None
    if not _sources_match(text):
        return None
    for name, g, mean in re.findall(r"<!-- trace (.+?) grid=(\d+) mean_us=([0-9.]+) -->", text):
        if name == kernel and int(g) == grid:
            return float(mean)
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--slots", type=int, default=4)
    p.add_argument("--no-rows", action="store_true", help="skip the per-row measurements of the other workloads")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--prewarm-ms", type=float, default=PREWARM_MS,
                   help="untimed steps run for this long before any loop is timed")
    p.add_argument("--reps", type=int, default=3,
                   help="timing windows inside the K timed steps (and repetitions of each per-launch loop); "
                        "the reported rates are their medians")
    p.add_argument("--trace-summary", metavar="DIR", help="only print the markdown summary of a rocprofv3 "
                   "--kernel-trace --output-format csv run written to DIR, and exit")
    p.add_argument("--pmc-summary", metavar="DIR", help="only print the markdown summary of rocprofv3 --pmc "
                   "--output-format csv runs written under DIR, and exit")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                   help="only run 10 device-to-device copies of MB megabytes (a plain copy kernel of known "
                        "size, used to scale the HBM traffic counters) and exit")
    return p.parse_args()


def copy_calibration(mb: int) -> None:
    import torch
    n = mb * 1000 * 1000
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_copy": n, "copies": 10}))


def main():
    args = parse()
    if args.trace_summary or args.pmc_summary:
        cmd = os.environ.get("PROFILE_COMMAND", "(command not recorded)")
        sys.stdout.write(trace_summary(args.trace_summary, cmd) if args.trace_summary
                         else pmc_summary(args.pmc_summary, cmd))
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path has no multi-GPU part",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_dequant_matrix_amd import qmv, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = synth.CONFIGS["c2"]
    N, K = c["N"], c["K"]
    Wg, Wu, x = synth.gate_up_problem()
    Ws, _ = synth.config_problem("c2")  # the plain product uses the gate-shape matrix of seed c2
    # slot sets: distinct device copies (the cache does not deduplicate)
    S = args.slots
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    slots = [(t(Ws), t(Wg), t(Wu)) for _ in range(S)]
    xd = t(x)
    y1 = torch.empty((1, N), device=dev)
    h = torch.empty((1, N), device=dev)
    wbytes = Ws.nbytes
    bytes_single = wbytes + K * 4 + N * 4
    bytes_pair = 2 * wbytes + K * 4 + N * 4
    bytes_step = bytes_single + bytes_pair

    def step(i):
        a, g, u = slots[i % S]
        qmv.qmv_q4_0(a, xd, y1, N, K, 1)
        qmv.qmv_q4_0_geglu(g, u, xd, h, N, K, 1)

    # The GPU reaches its sustained rate only after tens of milliseconds of
    # load (launch times fall by about 10% over the first 20 ms of back-to-back
    # GEMVs), so untimed steps run for --prewarm-ms first.
    t_end = time.perf_counter() + args.prewarm_ms * 1e-3
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(20):
            step(i)
            i += 1
        torch.cuda.synchronize()

    # per-kernel durations first: each entry point alone, back to back over
    # the slot sets, between one pair of events on the stream the kernels run
    # on (events between every launch would add their own queue packets),
    # repeated --reps times; the median repetition is reported.  They also
    # bring the GPU to its sustained-load clocks before the steps are timed.
    stream = torch.cuda.current_stream()

    def per_launch(fn, iters):
        for i in range(5):
            fn(i)
        reps = []
        for _ in range(args.reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for i in range(iters):
                fn(i)
            b.record(stream)
            torch.cuda.synchronize()
            reps.append(a.elapsed_time(b) / iters)
        return reps

    # The three matrices of every slot set have the same shape, so the
    # per-launch loops rotate over all 3 S of them (12 x 65 MB at S = 4, three
    # times the 256 MB last-level cache): the single matrix through each in
    # turn, the pair through the disjoint pairs (0, 1), (2, 3), ... of them, so
    # a matrix comes back only after all the others.
    mats = [m for sl in slots for m in sl]
    npairs = len(mats) // 2
    iters = max(args.steps // max(args.reps, 1), 1)
    t_single = per_launch(lambda i: qmv.qmv_q4_0(mats[i % len(mats)], xd, y1, N, K, 1), iters)
    t_pair = per_launch(lambda i: qmv.qmv_q4_0_geglu(mats[2 * (i % npairs)], mats[2 * (i % npairs) + 1],
                                                     xd, h, N, K, 1), iters)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # whole-step timing: exactly K steps between two synchronizations, split
    # into --reps windows by events on the kernels' stream
    nw = max(1, min(args.reps, args.steps))
    bounds = [args.steps * w // nw for w in range(nw + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nw + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for w in range(nw):
        for i in range(bounds[w], bounds[w + 1]):
            step(i)
        ev[w + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    windows = [ev[w].elapsed_time(ev[w + 1]) / (bounds[w + 1] - bounds[w]) for w in range(nw)]
    ms_step = _median(windows)
    ms_total = ev[0].elapsed_time(ev[nw]) / args.steps

    value = bytes_step / (ms_step * 1e-3) / 1e9
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    kernels = {}
    for entry, b, reps in (("qmv_q4_0", bytes_single, t_single), ("qmv_q4_0_geglu", bytes_pair, t_pair)):
        sym, per_cu = KERNEL_OF[entry]
        grid = unit_grid(N, K, cus, per_cu)
        tk = _median(reps)
        trace = profiled_trace_us(sym, grid)
        kernels[entry] = {"kernel": sym, "workgroups": grid, "bytes": b, "us": round(tk * 1e3, 3),
                          "us_reps": [round(r * 1e3, 3) for r in reps], "spread": round(_spread(reps), 4),
                          "GB/s": round(b / (tk * 1e-3) / 1e9, 1), "frac_of_hbm_peak": round(b / (tk * 1e-3) / 1e9 /
                                                                                          HBM_PEAK_GBS, 4),
                          "trace_us": trace, "us_over_trace": round(tk * 1e3 / trace, 4) if trace else None,
                          "hbm_traffic_bytes": profiled_traffic(sym, grid)}
    dom_entry, dom = max(kernels.items(), key=lambda kv: kv[1]["us"])
    roofline = {
        "bound": "hbm",
        "kernel": f"{dom_entry} ({dom['kernel']})",
        "achieved": dom["GB/s"],
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(dom["GB/s"] / HBM_PEAK_GBS, 4),
        "traffic": dom["hbm_traffic_bytes"],
        "traffic_source": TRAFFIC_PROFILE if dom["hbm_traffic_bytes"] is not None else None,
        "duration_source": f"median of {args.reps} back-to-back loops of {iters} launches, HIP events on the "
                           "launch stream",
        "trace_us": dom["trace_us"],
        "trace_source": TRACE_PROFILE if dom["trace_us"] is not None else None,
        "frac_from_trace": round(dom["bytes"] / (dom["trace_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        if dom["trace_us"] else None,
    }

    ceiling = read_ceiling(torch, qmv, dev, {"single": wbytes, "pair": 2 * wbytes})
    roofline["frac_of_read_ceiling"] = round(dom["GB/s"] / ceiling["pair"]["GB/s"], 4)

    rows = None
    if not args.no_rows:
        rows = measure_rows(torch, qmv, synth, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(synth, Ws, Wg, Wu, x, N, K, bytes_step, args.cpu_seconds)

    out = {
        "metric": "effective GB/s and % of HBM peak for fused-dequant Q4_0/Q8_0 GEMV, M=1",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_ms": args.prewarm_ms,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_windows": [round(w, 5) for w in windows],
        "window_spread": round(_spread(windows), 4),
        "ms_per_step_all_steps": round(ms_total, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded PCG64; Q4_0 d=|N(0,1)|*0.02, q~U{0..15}; x~N(0,1))",
        "config": {
            "workload": "Q4_0 GEMV 21504x5376 M=1 + gated GELU pair (two 21504x5376 Q4_0), one step = both",
            "weights": "Q4_0 (18-byte blocks of 32), dequantized in the kernel; f32 activations and accumulation",
            "N": N, "K": K, "M": 1, "bytes_per_step": bytes_step, "slot_sets": S,
            "working_set_MB": round(S * 3 * wbytes / 1e6, 1),
        },
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
        "read_ceiling": ceiling,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out))


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def _spread(v):
    """(max - min) / median of a list of timings."""
    return (max(v) - min(v)) / _median(v) if v else 0.0


def read_ceiling(torch, qmv, dev, sizes, iters=50):
    """The plain streaming-read rate (qmvdbg_stream_read: every byte loaded once
    with coalesced 16-byte loads) at the byte counts of the timed launches,
    over rotating buffers that add up to about 1 GB (4x the last-level cache)
    so that every read comes from HBM; the best of several grids."""
    out = {}
    word = torch.zeros(16384, dtype=torch.int32, device=dev)
    for name, nbytes in sizes.items():
        nbytes -= nbytes % 16
        copies = max(2 if nbytes >= 500_000_000 else 4, -(-1_000_000_000 // nbytes))
        bufs = [torch.full((nbytes,), i + 1, dtype=torch.uint8, device=dev) for i in range(copies)]
        best = None
        for wg in (256, 512, 768, 1024, 2048, 4096):
            ms = _time_loop(torch, lambda i: qmv.qmvdbg_stream_read(bufs[i % copies], nbytes, word, wg), iters)
            if best is None or ms < best[0]:
                best = (ms, wg)
        out[name] = {"bytes": nbytes, "copies": copies, "us": round(best[0] * 1e3, 2), "workgroups": best[1],
                     "GB/s": round(nbytes / (best[0] * 1e-3) / 1e9, 1)}
        del bufs
    return out


def _time_loop(torch, fn, iters, warm=5, reps=3):
    """Median over `reps` repetitions of the mean time (ms) of `iters`
    back-to-back calls, events on the current stream."""
    for i in range(warm):
        fn(i)
    out = []
    stream = torch.cuda.current_stream()
    for _ in range(reps):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(iters):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / iters)
    return _median(out)


def measure_rows(torch, qmv, synth, dev):
    """Effective GB/s of every other workload (context next to the headline)."""
    res = {}
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # C1: Q4_0 4096 x 4096, 64 slots (604 MB)
    c = synth.CONFIGS["c1"]
    W, x = synth.config_problem("c1")
    Wd = t(W)
    slots = [Wd.clone() for _ in range(64)]
    xd, y = t(x), torch.empty((1, c["N"]), device=dev)
    ms = _time_loop(torch, lambda i: qmv.qmv_q4_0(slots[i % 64], xd, y, c["N"], c["K"], 1), 200)
    b = W.nbytes + c["K"] * 4 + c["N"] * 4
    res["c1_qmv_q4_0_4096x4096"] = {"us": ms * 1e3, "bytes": b, "GB/s": b / ms / 1e6}
    del slots, Wd

    # C5: Q4_K 21504 x 5376, 8 slots
    c = synth.CONFIGS["c5"]
    W, x = synth.config_problem("c5")
    slots = [t(W) for _ in range(8)]
    xd, y = t(x), torch.empty((1, c["N"]), device=dev)
    ms = _time_loop(torch, lambda i: qmv.qmv_q4_k(slots[i % 8], xd, y, c["N"], c["K"], 1), 100)
    b = W.nbytes + c["K"] * 4 + c["N"] * 4
    res["c5_qmv_q4_k_21504x5376"] = {"us": ms * 1e3, "bytes": b, "GB/s": b / ms / 1e6}
    del slots

    # Q6_K at the FFN gate shape, and the FFN down shape (K = 21504) in Q6_K,
    # Q4_K and Q4_0, 8 slots each
    for name, fmt, entry in (("q6k_gate", "q6_k", qmv.qmv_q6_k), ("q6k_down", "q6_k", qmv.qmv_q6_k),
                             ("q4k_down", "q4_k", qmv.qmv_q4_k), ("c4", "q4_0", qmv.qmv_q4_0)):
        c = synth.CONFIGS[name]
        W, x = synth.config_problem(name, M=1)
        slots = [t(W) for _ in range(8)]
        xd, y = t(x), torch.empty((1, c["N"]), device=dev)
        ms = _time_loop(torch, lambda i: entry(slots[i % 8], xd, y, c["N"], c["K"], 1), 100)
        b = W.nbytes + c["K"] * 4 + c["N"] * 4
        res[f"{name}_qmv_{fmt}_{c['N']}x{c['K']}"] = {"us": ms * 1e3, "bytes": b, "GB/s": b / ms / 1e6}
        if name.endswith("down"):
            # the same product with the GELU gate folded into its input (reads g and u)
            ud = t(synth.activations(1, c["K"], synth.SEEDS[name] + 1))
            gated = getattr(qmv, f"qmv_{fmt}_geglu_down")
            ms = _time_loop(torch, lambda i: gated(slots[i % 8], xd, ud, y, c["N"], c["K"], 1), 100)
            b = W.nbytes + 2 * c["K"] * 4 + c["N"] * 4
            res[f"{name}_qmv_{fmt}_geglu_down_{c['N']}x{c['K']}"] = {"us": ms * 1e3, "bytes": b,
                                                                   "GB/s": b / ms / 1e6}
        del slots

    # MXFP4 (codes and E8M0 scales in two planes) at the gate and down shapes, 8 slots
    for name in ("mxfp4_gate", "mxfp4_down"):
        c = synth.CONFIGS[name]
        codes, scales, x = synth.mxfp4_problem(c["N"], c["K"], 1, synth.SEEDS[name])
        sl = [(t(codes), t(scales)) for _ in range(8)]
        xd, y = t(x), torch.empty((1, c["N"]), device=dev)
        ms = _time_loop(torch, lambda i: qmv.qmv_mxfp4(*sl[i % 8], xd, y, c["N"], c["K"], 1), 100)
        b = codes.nbytes + scales.nbytes + c["K"] * 4 + c["N"] * 4
        res[f"{name}_qmv_mxfp4_{c['N']}x{c['K']}"] = {"us": ms * 1e3, "bytes": b, "GB/s": b / ms / 1e6}
        del sl

    # Attention projections of a Q4_K_M model (Q, K in Q4_K, V in Q6_K): one
    # launch, and the three single-matrix launches it replaces; 16 slots
    # (442 MB, past the 256 MB last-level cache)
    c = synth.CONFIGS["qkv"]
    Wq, Wk, Wv, x = synth.qkv_problem()
    sl = [(t(Wq), t(Wk), t(Wv)) for _ in range(16)]
    xd = t(x)
    yq, yk, yv = (torch.empty((1, n), device=dev) for n in (c["Nq"], c["Nk"], c["Nv"]))
    K = c["K"]
    b = Wq.nbytes + Wk.nbytes + Wv.nbytes + K * 4 + (c["Nq"] + c["Nk"] + c["Nv"]) * 4
    ms = _time_loop(torch, lambda i: qmv.qmv_q4_k_q6_k_qkv(*sl[i % 16], xd, yq, yk, yv, c["Nq"], c["Nk"], c["Nv"],
                                                          K, 1), 200)
    res["qkv_q4_k_q6_k_4096+2048+2048x5376_one_launch"] = {"us": ms * 1e3, "bytes": b, "GB/s": b / ms / 1e6}

    def three(i):
        a, k_, v_ = sl[i % 16]
        qmv.qmv_q4_k(a, xd, yq, c["Nq"], K, 1)
        qmv.qmv_q4_k(k_, xd, yk, c["Nk"], K, 1)
        qmv.qmv_q6_k(v_, xd, yv, c["Nv"], K, 1)
    ms = _time_loop(torch, three, 200)
    res["qkv_q4_k_q6_k_4096+2048+2048x5376_three_launches"] = {"us": ms * 1e3, "bytes": b, "GB/s": b / ms / 1e6}
    del sl

    # C4: Q4_0 x Q8 activations, 5376 x 21504, M = 1, 16, 512; 8 slots
    c = synth.CONFIGS["c4"]
    N, K = c["N"], c["K"]
    W, _ = synth.config_problem("c4", M=1)
    slots = [t(W) for _ in range(8)]
    for M in c["Ms"]:
        x = synth.activations(M, K, synth.SEEDS["c4"])
        xd, y = t(x), torch.empty((M, N), device=dev)
        wsb = qmv.qmm_q4_0_q8act_ws_bytes(N, K, M)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        iters = 100 if M < 512 else 20
        ms = _time_loop(torch, lambda i: qmv.qmm_q4_0_q8act(slots[i % 8], xd, y, N, K, M, ws, wsb), iters,
                        warm=2 if M < 512 else 10)
        b = W.nbytes + M * K * 4 + M * N * 4
        res[f"c4_qmm_q4_0_q8act_M{M}"] = {"us": ms * 1e3, "bytes": b, "GB/s": b / ms / 1e6,
                                          "int_TOPS": 2.0 * M * N * K / ms / 1e9}
    del slots

    # Q4_0 x float32 activations, a few rows at once, on the 21504 x 5376 FFN
    # matrix (8 slots): the fixed-eight verifier batch and the 32-row prefill
    # tile, next to the same rows through the matrix-vector kernel row by row
    c = synth.CONFIGS["c2"]
    N, K = c["N"], c["K"]
    W, _ = synth.config_problem("c2")
    slots = [t(W) for _ in range(8)]
    for M in (8, 32):
        x = synth.activations(M, K, 2100 + M)
        xd, y = t(x), torch.empty((M, N), device=dev)
        wsb = qmv.qmm_q4_0_f32act_ws_bytes(N, K, M)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        ms = _time_loop(torch, lambda i: qmv.qmm_q4_0_f32act(slots[i % 8], xd, y, N, K, M, ws, wsb), 100, warm=3)
        b = W.nbytes + M * K * 4 + M * N * 4
        res[f"c2_qmm_q4_0_f32act_M{M}"] = {"us": ms * 1e3, "bytes": b, "GB/s": b / ms / 1e6,
                                           "TFLOPS": 2.0 * M * N * K / ms / 1e9}
        if M == 8:
            ms = _time_loop(torch, lambda i: qmv.qmv_q4_0(slots[i % 8], xd, y, N, K, M), 30, warm=2)
            res["c2_qmv_q4_0_rowwise_M8"] = {"us": ms * 1e3, "bytes": b, "GB/s": b / ms / 1e6}
    del slots

    # C3: Q8_0 262144 x 5376 + soft-cap + top-10 (1.5 GB: one copy streams)
    c = synth.CONFIGS["c3"]
    W, x = synth.config_problem("c3")
    Wd, xd = t(W), t(x)
    del W
    k = c["k"]
    wsb = qmv.logits_topk_ws_bytes(c["N"], 1, k)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    vals = torch.empty((1, k), device=dev)
    idx = torch.empty((1, k), dtype=torch.int32, device=dev)
    ms = _time_loop(torch, lambda i: qmv.logits_topk(Wd, xd, vals, idx, c["N"], c["K"], 1, k, c["softcap"], ws,
                                                     wsb), 20, warm=3)
    b = Wd.numel() + c["K"] * 4 + c["N"] * 4
    res["c3_logits_topk_q8_0_262144x5376_k10"] = {"us": ms * 1e3, "bytes": b, "GB/s": b / ms / 1e6}
    # gap between the k-th and (k+1)-th logit (the index set is unique when it
    # exceeds twice the float tolerance); the logits are left in the workspace
    ylog = ws[: c["N"] * 4].view(torch.float32)
    top = torch.topk(ylog.double(), k + 1).values
    res["c3_kth_logit_margin"] = {"value": float(top[k - 1] - top[k]), "seed": synth.SEEDS["c3"]}
    y = torch.empty((1, c["N"]), device=dev)
    ms = _time_loop(torch, lambda i: qmv.qmv_q8_0(Wd, xd, y, c["N"], c["K"], 1), 20, warm=3)
    res["c3_qmv_q8_0_only_262144x5376"] = {"us": ms * 1e3, "bytes": b, "GB/s": b / ms / 1e6}
    c3_weight_bytes = Wd.numel()
    # token selection on the device: top-40, then a top-p draw (0.95, T = 1)
    k40 = 40
    wsb40 = qmv.logits_topk_ws_bytes(c["N"], 1, k40)
    ws40 = torch.empty(wsb40, dtype=torch.uint8, device=dev)
    v40 = torch.empty((1, k40), device=dev)
    i40 = torch.empty((1, k40), dtype=torch.int32, device=dev)
    ud = torch.full((1,), 0.5, device=dev)
    tok = torch.empty((1,), dtype=torch.int32, device=dev)
    nuc = torch.empty((1,), dtype=torch.int32, device=dev)
    ms = _time_loop(torch, lambda i: qmv.logits_sample(Wd, xd, ud, tok, nuc, v40, i40, c["N"], c["K"], 1, k40,
                                                       c["softcap"], 1.0, 0.95, ws40, wsb40), 20, warm=3)
    res["c3_logits_sample_q8_0_262144x5376_k40_p0.95"] = {"us": ms * 1e3, "bytes": b, "GB/s": b / ms / 1e6}
    # the two-stage top-k alone, on the same logits
    yl = ylog.clone().reshape(1, -1)
    ms = _time_loop(torch, lambda i: qmv.qmvdbg_topk_f32(yl, vals, idx, c["N"], 1, k, c["softcap"], ws, wsb), 50,
                    warm=3)
    res["c3_topk_only_262144_k10"] = {"us": ms * 1e3, "bytes": c["N"] * 4, "GB/s": c["N"] * 4 / ms / 1e6}
    del Wd
    # the 1024-wide drafter projection over the same vocabulary (Q8_0 262144 x 1024) + selection; four
    # rotating copies (1.1 GB, 4x the last-level cache), so that the weights come from HBM
    Kd = 1024
    Wm = [t(synth.q8_0_weights(c["N"], Kd, 1103))]
    Wm += [Wm[0].clone() for _ in range(3)]
    xm = t(synth.activations(1, Kd, 1104))
    ms = _time_loop(torch, lambda i: qmv.logits_sample(Wm[i % 4], xm, ud, tok, nuc, v40, i40, c["N"], Kd, 1, k40,
                                                       c["softcap"], 1.0, 0.95, ws40, wsb40), 50, warm=3)
    bm = Wm[0].numel() + Kd * 4 + c["N"] * 4
    res["mtp_logits_sample_q8_0_262144x1024_k40_p0.95"] = {"us": ms * 1e3, "bytes": bm, "GB/s": bm / ms / 1e6}
    ms = _time_loop(torch, lambda i: qmv.qmv_q8_0(Wm[i % 4], xm, y, c["N"], Kd, 1), 50, warm=3)
    res["mtp_qmv_q8_0_only_262144x1024"] = {"us": ms * 1e3, "bytes": bm, "GB/s": bm / ms / 1e6}
    mtp_weight_bytes = Wm[0].numel()
    del Wm
    # the plain streaming read at the logit projections' weight sizes, next to their GEMV rates
    ceil = read_ceiling(torch, qmv, dev, {"c3": c3_weight_bytes, "mtp": mtp_weight_bytes}, iters=20)
    res["read_ceiling_logits"] = ceil
    for row, key in (("c3_qmv_q8_0_only_262144x5376", "c3"), ("mtp_qmv_q8_0_only_262144x1024", "mtp")):
        res[row]["frac_of_read_ceiling"] = round(res[row]["GB/s"] / ceil[key]["GB/s"], 4)
    # a plain device-to-device copy of 256 MB (read + write), next to the GEMV rates
    a = torch.empty(256 * 1000 * 1000, dtype=torch.uint8, device=dev).fill_(1)
    bb = torch.empty_like(a)
    ms = _time_loop(torch, lambda i: bb.copy_(a), 20, warm=3)
    res["copy_256MB_read_plus_write"] = {"us": ms * 1e3, "bytes": 2 * a.numel(), "GB/s": 2 * a.numel() / ms / 1e6}
    del a, bb
    for v in res.values():
        if "GB/s" in v:
            v["frac_of_hbm_peak"] = v["GB/s"] / HBM_PEAK_GBS
        if "int_TOPS" in v:
            v["frac_of_int8_mfma_peak"] = v["int_TOPS"] / INT8_MFMA_PEAK_TOPS
        for key in list(v):
            if isinstance(v[key], float):
                v[key] = round(v[key], 4 if key.startswith("frac") else 2)
    return res


def cpu_baseline(synth, Ws, Wg, Wu, x, N, K, bytes_step, seconds):
    """The float64 oracle on the host cores, timed on whole steps of the same
    workload (one plain product and the gated pair) until `seconds` pass."""
    import oracle
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.qmv("q4_0", Ws, N, K, x)
        g, _ = oracle.qmv("q4_0", Wg, N, K, x)
        u, _ = oracle.qmv("q4_0", Wu, N, K, x)
        oracle.geglu(g, u)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    cores = oracle.num_threads()
    # the 4096 x 4096 workload single-threaded, for reference
    c1W, c1x = synth.config_problem("c1")
    oracle.set_num_threads(1)
    t1 = time.perf_counter()
    oracle.qmv("q4_0", c1W, 4096, 4096, c1x)
    t1 = time.perf_counter() - t1
    oracle.set_num_threads(cores)
    return {
        "value": round(bytes_step * reps / el / 1e9, 3),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{reps} whole steps (3 x 21504x5376 Q4_0 matrices each) in {el:.1f} s, float64, OpenMP",
        "c1_4096x4096_single_thread_s": round(t1, 4),
        "cpu_model": _cpu_model(),
    }


# ------------------------------------------------------------ profile summaries
# Sources whose sha256 is recorded in a summary: the numbers in it are valid
# while these are unchanged.
PROFILED_SOURCES = ("quantized_dequant_matrix_amd/csrc/gemv.hip", "quantized_dequant_matrix_amd/csrc/qmm.hip",
                    "quantized_dequant_matrix_amd/csrc/topk.hip", "quantized_dequant_matrix_amd/csrc/stream.hip",
                    "quantized_dequant_matrix_amd/csrc/qmv_device.h", "quantized_dequant_matrix_amd/build.py")


def _kernel_symbol(name: str) -> str:
    """'void qmv::(anonymous namespace)::k<1, 2>(args)' -> 'qmv::k<1, 2>'."""
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def _csv_rows(directory: str, suffix: str, calibration=None):
    """Rows of every rocprofv3 CSV named *suffix under directory; with
    calibration True / False only those of runs written with -o cal /
    the others."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        if calibration is not None and os.path.basename(path).startswith("cal") != calibration:
            continue
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _workgroups(r) -> int:
    grid = int(r.get("Grid_Size") or r.get("Grid_Size_X") or 0)
    wg = int(r.get("Workgroup_Size") or r.get("Workgroup_Size_X") or 1)
    return grid // max(wg, 1)


def _source_lines():
    import hashlib
    out = ["Sources the numbers were taken on (sha256):", ""]
    for src in PROFILED_SOURCES:
        with open(os.path.join(ROOT, src), "rb") as f:
            out.append(f"- source_sha256 {src} {hashlib.sha256(f.read()).hexdigest()}")
    return out


def trace_summary(directory: str, command: str, warm_ms: float = PREWARM_MS) -> str:
    """Markdown table of a rocprofv3 --kernel-trace run: per kernel and grid,
    calls and mean / median / min / max durations, the mean of the calls that
    start warm_ms or more after that kernel's first call (bench.py times its
    loops after that long a warm-up), plus a machine-readable line per kernel
    that profiled_trace_us() reads (the warm mean where there are such calls)."""
    import statistics
    groups = {}
    for r in _csv_rows(directory, "kernel_trace.csv"):
        key = (_kernel_symbol(r["Kernel_Name"]), _workgroups(r))
        start, end = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        groups.setdefault(key, []).append((start, (end - start) / 1000.0))
    lines = ["# Kernel trace of bench.py: every kernel the command below launches", "",
             "Command (from the repository root, one MI355X):", "", "```", command, "```", "",
             "Durations from the kernel trace, per kernel symbol and grid (workgroups). \"warm\" counts the",
             f"calls that start {warm_ms:g} ms or more after the kernel's first call (bench.py's loops are timed",
             "after that long a warm-up); kernels that run for less have none.", "",
             "| kernel | grid | calls | mean us | median us | min us | max us | warm calls | warm mean us |",
             "|---|---|---|---|---|---|---|---|---|"]
    marks = []
    for (k, g), calls in sorted(groups.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        v = [d for _, d in calls]
        first = min(s for s, _ in calls)
        warm = [d for s, d in calls if s >= first + warm_ms * 1e6]
        wm = statistics.mean(warm) if warm else None
        lines.append(f"| `{k}` | {g} | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} | "
                     f"{min(v):.2f} | {max(v):.2f} | {len(warm)} | {f'{wm:.2f}' if warm else '-'} |")
        marks.append(f"<!-- trace {k} grid={g} mean_us={(wm if warm else statistics.mean(v)):.3f} -->")
    return "\n".join(lines + [""] + _source_lines() + [""] + marks) + "\n"


def pmc_summary(directory: str, command: str) -> str:
    """Markdown table of rocprofv3 --pmc runs (every run_counter_collection.csv
    under `directory`): per kernel and grid, the median of each counter over
    its dispatches.  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled
    by what they read for the plain copies of bench.py --copy-calibration
    (bytes per copy known), and written as machine-readable traffic lines."""
    import statistics
    def medians(rows):
        vals = {}
        for r in rows:
            key = (_kernel_symbol(r["Kernel_Name"]), _workgroups(r))
            vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        return {k: {c: statistics.median(v) for c, v in cs.items()} for k, cs in vals.items()}

    med = medians(_csv_rows(directory, "counter_collection.csv", calibration=False))
    counters = sorted({c for cs in med.values() for c in cs})
    # calibration runs (-o cal): bench.py --copy-calibration 256, ten device
    # copies of 256 MB (256e6 bytes read and written per dispatch)
    cal = {}
    for (k, g), cs in medians(_csv_rows(directory, "counter_collection.csv", calibration=True)).items():
        if "copy" in k.lower():
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                if c in cs and cs[c] > 0:
                    cal[c] = 256e6 / (cs[c] * 1024.0)
    lines = ["# Counters of bench.py's kernels (rocprofv3 --pmc)", "", "Commands (from the repository root, one "
             "MI355X):", "", "```", command, "```", "", "Medians over each kernel's dispatches:", "",
             "| kernel | grid | " + " | ".join(counters) + " |", "|---|---|" + "---|" * len(counters)]
    marks = []
    for (k, g), cs in sorted(med.items(), key=lambda kv: -kv[1].get("FETCH_SIZE", kv[1].get("SQ_WAVES", 0))):
        lines.append(f"| `{k}` | {g} | " + " | ".join(f"{cs[c]:.6g}" if c in cs else "" for c in counters) + " |")
        if "FETCH_SIZE" in cs and "WRITE_SIZE" in cs and cal.get("FETCH_SIZE") and cal.get("WRITE_SIZE"):
            rd = cs["FETCH_SIZE"] * 1024.0 * cal["FETCH_SIZE"]
            wr = cs["WRITE_SIZE"] * 1024.0 * cal["WRITE_SIZE"]
            marks.append(f"<!-- traffic {k} grid={g} read={rd:.0f} write={wr:.0f} -->")
    if cal:
        lines += ["", "Copy calibration (bytes per KiB counted): " +
                  ", ".join(f"{c} x{cal[c] * 1024.0:.1f}" for c in sorted(cal))]
    return "\n".join(lines + [""] + _source_lines() + [""] + marks) + "\n"


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the persistent tiled GEMM (8192^3 bf16, bf16 C) per tile
scheduler, plus the persistent fp32 add, on one MI355X.

Prints ONE JSON line.  `value` is the GEMM throughput (TFLOP/s) of the
work-stealing scheduler on the 8192^3 workload; every scheduler's figure, the
add's GB/s, the roofline of the dominant kernel and the CPU oracle baseline
are reported in the same line.

Timed region: W untimed warm-up steps, then exactly K steps bracketed by
torch.cuda.synchronize() on both sides; inputs are resident in HBM before the
timed region starts.  A step is one pgemm_run call (counter reset + persistent
GEMM launch) on the stream the library launches on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_CLOCK_GHZ = 2.4          # engine clock the dense peak is quoted at
M = N = K = 8192
SCHEDS = [("blocked", 8, 0), ("interleaved", 8, 0), ("grouped", 8, 0), ("grouped", 16, 0),
          ("work_stealing", 8, 0), ("work_stealing", 16, 0), ("blocked_grouped", 8, 0), ("stream_k", 8, 0),
          ("work_stealing_xcc", 8, 0), ("work_stealing", 8, -1), ("work_stealing_xcc", 8, -1)]
HEADLINE = ("work_stealing", 8)   # key work_stealing_g8: one tile per claim, as on the pages
CPU_ROWS = 4096
SETTLE_S = 2.0        # untimed repeats of the headline call before the timed steps (engine clock settles)
RAGGED_ROUNDS = 3     # interleaved rounds over the schedulers on the ragged shapes
ROOFLINE_SETTLE_S = 0.4  # untimed repeats of a short kernel before each of its timed batches

# Memory traffic of one launch: what the L2s send to the memory controllers,
# from rocprofv3 counter passes over `bench.py --profile-only <target>`:
# TCC_EA0_RDREQ_DRAM_32B_sum and TCC_EA0_WRREQ_WRITE_DRAM_32B_sum (32-byte
# units of read and write requests bound for the memory controllers, a
# 128-byte request counting 4; median of the 9 dispatches of a pass) x 32 bytes.
# On a plain 256 MiB device copy (`bench.py --copy-calibration`) they read
# exactly 256 MiB each way, so no calibration factor applies.  Hits in the
# Infinity Cache, which sits on the memory side, are included: no counter
# here separates them from DRAM.  A record holds only for the kernel sources
# it was measured on (hash); otherwise the traffic is reported as null.
# (runtime.hip decides each launch's grid, program numbering and group size)
BF16_SOURCES = ["gemm_bf16_lds.hip", "gemm_device.hpp", "common.hpp", "sched.hpp", "runtime.hip"]
FP8_SOURCES = ["gemm_fp8.hip", "gemm_device.hpp", "common.hpp", "sched.hpp", "runtime.hip"]
ADD_SOURCES = ["padd.hip", "common.hpp", "sched.hpp", "runtime.hip"]
TRAFFIC = {
    "bf16_8192cube_work_stealing": {"sources": BF16_SOURCES, "sha256_16": "6ad34d738c399914",
        "read_bytes": 1610946752, "write_bytes": 186131840},
    "fp8_8192cube_work_stealing": {"sources": FP8_SOURCES, "sha256_16": "c29722996871b668",
        "read_bytes": 811933376, "write_bytes": 144911136},
    "fp8_256x28672x8192_128x256_work_stealing": {"sources": FP8_SOURCES, "sha256_16": "c29722996871b668",
        "read_bytes": 253829248, "write_bytes": 14680320},
    "fp8_256x28672x8192_128x256_grouped": {"sources": FP8_SOURCES, "sha256_16": "c29722996871b668",
        "read_bytes": 253793792, "write_bytes": 14680064},
    "add_8192sq_128x128_blocked": {"sources": ADD_SOURCES, "sha256_16": "e9c3685c3537e947",
        "read_bytes": 536905728, "write_bytes": 268644352},
    "add_8192sq_128x128_work_stealing": {"sources": ADD_SOURCES, "sha256_16": "e9c3685c3537e947",
        "read_bytes": 536960000, "write_bytes": 268485120},
    "add_8192sq_32x16_blocked": {"sources": ADD_SOURCES, "sha256_16": "e9c3685c3537e947",
        "read_bytes": 1073797120, "write_bytes": 268435456},
    "add_8192sq_32x16_work_stealing": {"sources": ADD_SOURCES, "sha256_16": "e9c3685c3537e947",
        "read_bytes": 536980160, "write_bytes": 320627072},
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default="", help="comma list of schedulers (or keys such as work_stealing_g8) to time (profiling runs)")
    p.add_argument("--skip-add", action="store_true")
    p.add_argument("--skip-extra", action="store_true", help="only the 8192^3 bf16 GEMM and the add")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only time a plain 256 MiB device-to-device copy (the reference kernel for "
                        "scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    p.add_argument("--profile-only", choices=sorted(PROFILE_TARGETS), default=None,
                   help="only time this one workload (for traces and counter passes) and exit")
    p.add_argument("--settle", type=float, default=SETTLE_S,
                   help="with --profile-only: seconds of untimed calls first (0 for counter passes)")
    return p.parse_args()


# Single workloads for counter passes: name -> (kind, tile, scheduler[, pipeline]).
PROFILE_TARGETS = {
    # the headline workload (A, B normal(0,1) from seeds 1030 / 1031)
    "bf16_8192cube_work_stealing": ("bf16n:8192:8192:8192", (256, 256, 64), "work_stealing"),
    "bf16_8192cube_work_stealing_pingpong": ("bf16n:8192:8192:8192", (256, 256, 64), "work_stealing", "pingpong"),
    "bf16_8192cube_work_stealing_four_wave": ("bf16n:8192:8192:8192", (256, 256, 64), "work_stealing", "four_wave"),
    "bf16_8192cube_grouped": ("bf16n:8192:8192:8192", (256, 256, 64), "grouped"),
    "bf16_8192cube_interleaved": ("bf16n:8192:8192:8192", (256, 256, 64), "interleaved"),
    "torch_bf16_8192cube": ("bf16n:8192:8192:8192", None, "torch"),
    # the same shape on separate all-zero A and B: operands that draw little
    # power, so the chip holds its full clock (the kernel's own ceiling)
    "bf16_8192cube_zeros_work_stealing": ("bf16z:8192:8192:8192", (256, 256, 64), "work_stealing"),
    "bf16_8192cube_zeros_grouped": ("bf16z:8192:8192:8192", (256, 256, 64), "grouped"),
    "torch_bf16_8192cube_zeros": ("bf16z:8192:8192:8192", None, "torch"),
    "bf16_512cube_fp32_blocked": ("bf16f:512:512:512", (128, 128, 64), "blocked"),
    "add_8192sq_128x128_blocked": ("add", (128, 128), "blocked"),
    "add_8192sq_128x128_work_stealing": ("add", (128, 128), "work_stealing"),
    "add_8192sq_32x16_work_stealing": ("add", (32, 16), "work_stealing"),
    "add_8192sq_32x16_blocked": ("add", (32, 16), "blocked"),
    "add_8192sq_32x16_interleaved": ("add", (32, 16), "interleaved"),
    "add_8192sq_128x128_interleaved": ("add", (128, 128), "interleaved"),
    "fp8_8192cube_work_stealing": ("fp8", (256, 256, 128), "work_stealing"),
    "fp8_256x28672x8192_128x256_work_stealing": ("fp8_skinny", (128, 256, 128), "work_stealing"),
    "fp8_256x28672x8192_128x256_grouped": ("fp8_skinny", (128, 256, 128), "grouped"),
    "fp8_256x28672x8192_128x256_stream_k": ("fp8_skinny", (128, 256, 128), "stream_k"),
    # ragged bf16 shapes (same inputs as the bench pass) at the default,
    # balanced grid and, with "_grid256", on one program per CU
    "bf16_5120x5120x4096_work_stealing": ("bf16:5120:5120:4096", (256, 256, 64), "work_stealing"),
    "bf16_5120x5120x4096_work_stealing_grid256": ("bf16:5120:5120:4096:256", (256, 256, 64), "work_stealing"),
    "bf16_5120x5120x4096_blocked_grouped": ("bf16:5120:5120:4096", (256, 256, 64), "blocked_grouped"),
    "bf16_4864x8000x8192_work_stealing": ("bf16:4864:8000:8192", (256, 256, 64), "work_stealing"),
    "bf16_4864x8000x8192_work_stealing_grid256": ("bf16:4864:8000:8192:256", (256, 256, 64), "work_stealing"),
    "bf16_3000x7000x2048_work_stealing": ("bf16:3000:7000:2048", (256, 256, 64), "work_stealing"),
    "bf16_3000x7000x2048_work_stealing_grid256": ("bf16:3000:7000:2048:256", (256, 256, 64), "work_stealing"),
    "bf16_4864x8000x8192_grouped": ("bf16:4864:8000:8192", (256, 256, 64), "grouped"),
    "bf16_4864x8000x8192_blocked_grid256": ("bf16:4864:8000:8192:256", (256, 256, 64), "blocked"),
    "bf16_4864x8000x8192_grouped_grid256": ("bf16:4864:8000:8192:256", (256, 256, 64), "grouped"),
    "bf16_3000x7000x2048_blocked": ("bf16:3000:7000:2048", (256, 256, 64), "blocked"),
    "bf16_3000x7000x2048_blocked_grid256": ("bf16:3000:7000:2048:256", (256, 256, 64), "blocked"),
    "bf16_3000x7000x2048_interleaved_grid256": ("bf16:3000:7000:2048:256", (256, 256, 64), "interleaved"),
    # stream-K (main kernel and fix-up) on the ragged and the under-filled shapes
    "bf16_5120x5120x4096_stream_k": ("bf16:5120:5120:4096", (256, 256, 64), "stream_k"),
    "bf16_4864x8000x8192_stream_k": ("bf16:4864:8000:8192", (256, 256, 64), "stream_k"),
    "bf16_3000x7000x2048_stream_k": ("bf16:3000:7000:2048", (256, 256, 64), "stream_k"),
    "bf16_8192x1024x8192_stream_k": ("bf16:8192:1024:8192", (256, 256, 64), "stream_k"),
    "bf16_1024x8192x8192_stream_k": ("bf16:1024:8192:8192", (256, 256, 64), "stream_k"),
    "bf16_2048x2048x8192_stream_k": ("bf16:2048:2048:8192", (256, 256, 64), "stream_k"),
    "bf16_8192x1024x8192_work_stealing": ("bf16:8192:1024:8192", (256, 256, 64), "work_stealing"),
    "bf16_2048x2048x8192_work_stealing": ("bf16:2048:2048:8192", (256, 256, 64), "work_stealing"),
}


def profile_only(name, steps, warmup, settle_s):
    """Time one workload of the bench pass (same inputs) and print its event
    time, so that a trace or counter pass sees only that kernel: settle_s
    seconds of untimed calls (the engine clock settles, as in the bench
    pass), then warmup and steps calls."""
    import torch
    import tile_scheduling_persistent_amd as pg
    from synthetic import f32_normal, fp8_blockscaled
    kind, tile, sched = PROFILE_TARGETS[name][:3]
    pipeline = PROFILE_TARGETS[name][3] if len(PROFILE_TARGETS[name]) > 3 else "default"
    cfg = pg.Config(0)
    stream = torch.cuda.current_stream()
    if kind.split(":")[0] in ("bf16", "bf16n", "bf16f", "bf16z"):
        from synthetic import bf16_bits_normal, bf16_bits_uniform
        dims = [int(x) for x in kind.split(":")[1:]]
        m, n, k = dims[:3]
        grid = dims[3] if len(dims) > 3 else 0
        if kind.startswith("bf16n:"):
            ab = bf16_bits_normal((m, k), 1030), bf16_bits_normal((k, n), 1031)
        elif kind.startswith("bf16z:"):
            ab = np.zeros((m, k), np.uint16), np.zeros((k, n), np.uint16)
        elif kind.startswith("bf16f:"):
            ab = bf16_bits_uniform((m, k), 1010), bf16_bits_uniform((k, n), 1011)
        else:
            ab = bf16_bits_uniform((m, k), 1040 + m), bf16_bits_uniform((k, n), 1041 + n)
        ra = torch.from_numpy(ab[0].view(np.int16)).to("cuda:0").view(torch.bfloat16)
        rb = torch.from_numpy(ab[1].view(np.int16)).to("cuda:0").view(torch.bfloat16)
        out = "bf16_out_f32" if kind.startswith("bf16f:") else "bf16_out_bf16"
        rc = torch.empty((m, n), dtype=torch.float32 if out == "bf16_out_f32" else torch.bfloat16, device="cuda:0")
        nbytes, work = 2 * (m * k + k * n) + rc.element_size() * m * n, 2.0 * m * n * k
        if sched == "torch":  # hipBLASLt on the same operands, for comparison
            a = None
            fn = lambda: torch.matmul(ra, rb, out=rc)  # noqa: E731
        else:
            a = pg.make_args(tile=tile, grid=grid, pipeline=pipeline)
            fn = lambda: pg.pgemm_run(cfg, ra, rb, rc, m, n, k, out, sched, a)  # noqa: E731
    elif kind == "add":
        R = Cc = 8192
        X = torch.from_numpy(f32_normal((R, Cc), 2001)).to("cuda:0")
        Y = torch.from_numpy(f32_normal((R, Cc), 2002)).to("cuda:0")
        Z = torch.empty_like(X)
        nbytes, work = 3 * R * Cc * 4, None
        fn = lambda: pg.padd_run(cfg, X, Y, Z, R, Cc, tile[0], tile[1], sched)  # noqa: E731
    else:
        m, n, k = (8192, 8192, 8192) if kind == "fp8" else (256, 28672, 8192)
        qa, sa = fp8_blockscaled(m, k, 1050, 1052, k_major=True)
        qb, sb = fp8_blockscaled(n, k, 1051, 1053, k_major=False)
        dA, dB = torch.from_numpy(qa).to("cuda:0"), torch.from_numpy(qb).to("cuda:0")
        dSA, dSB = torch.from_numpy(sa).to("cuda:0"), torch.from_numpy(sb).to("cuda:0")
        dC = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
        a = pg.make_args(tile=tile, a_scale=dSA, b_scale=dSB)
        nbytes, work = m * k + k * n + (m + n) * (k // 128) + 2 * m * n, 2.0 * m * n * k
        fn = lambda: pg.pgemm_run(cfg, dA, dB, dC, m, n, k, "fp8_b128_out_bf16", sched, a)  # noqa: E731
    settle(fn, settle_s)
    d = event_means(fn, steps, warmup, stream)
    batch = event_batch_ms(fn, steps, 2, stream)
    ev_mean = float(np.mean(d))
    out = {"profile_only": name, "event_ms_mean": round(ev_mean, 5), "event_ms_median": round(float(np.median(d)), 5),
           "batch_ms_per_call": round(batch, 5),
           "plan": (pg.plan_gemm(cfg, m, n, k, "bf16_out_f32" if kind.startswith("bf16f:") else "bf16_out_bf16",
                                 sched, a) if kind.split(":")[0] in ("bf16", "bf16n", "bf16f", "bf16z")
                   and sched != "torch" else None),
           "algorithmic_bytes": nbytes, "gbs": round(nbytes / (ev_mean * 1e-3) / 1e9, 1)}
    if work:
        out["tflops"] = round(work / (ev_mean * 1e-3) / 1e12, 2)
    print(json.dumps(out), flush=True)


def copy_calibration(steps, warmup):
    """A plain copy of a 256 MiB fp32 buffer: reads 256 MiB and writes 256 MiB
    per launch, so a counter pass over it gives the factor between what the
    counter reports and the bytes actually moved."""
    import torch
    n = 64 * 1024 * 1024
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    ms, ev_mean, _ = time_calls(lambda: dst.copy_(src), steps, warmup, stream)
    print(json.dumps({"copy_calibration": {"bytes_read": 4 * n, "bytes_written": 4 * n,
                                           "event_ms_mean": round(ev_mean, 5),
                                           "gbs": round(8 * n / (ev_mean * 1e-3) / 1e9, 1)}}), flush=True)


def settle(fn, seconds):
    """Repeat `fn` (untimed) for `seconds`: the engine clock under a sustained
    load is lower than at the first launches, and the timed steps should see
    the sustained clock."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def event_means(fn, steps, warmup, stream):
    """Per-call HIP-event durations (ms) of `steps` calls after `warmup`."""
    import torch
    for _ in range(warmup):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def event_batch_ms(fn, steps, warmup, stream):
    """Mean time per call (ms) of `steps` calls enqueued back to back between
    one pair of HIP events on `stream`.  The warm-up calls go right before the
    first event, so the GPU is busy while the host enqueues the timed calls;
    for kernels longer than the host's cost per call the GPU then runs them
    back to back, and the mean is the kernel time plus the gap between
    consecutive launches (per-call event pairs add their own commands to that
    gap)."""
    import torch
    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def graph_ms_per_call(fn, calls, replays, stream):
    """Mean time per call (ms) of `calls` calls captured in one HIP graph,
    median over `replays` replays: the launch rate the device sustains when
    the host's cost per call is out of the way (for kernels shorter than that
    cost).  Only for calls that record no memset into the graph."""
    import torch
    g = torch.cuda.CUDAGraph()
    fn()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / calls)
    del g
    return float(np.median(out))


def rounds_summary(work, means_ms, unit_scale=1e12):
    """Median / min / max rate over rounds (work per call / mean call time)."""
    rates = sorted(work / (m * 1e-3) / unit_scale for m in means_ms)
    return {"median": round(float(np.median(rates)), 2), "min": round(rates[0], 2),
            "max": round(rates[-1], 2), "rounds": len(rates)}


def time_calls(fn, steps, warmup, stream):
    """Wall time of `steps` calls plus per-call HIP-event durations on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs = [e0.elapsed_time(e1) for e0, e1 in evs]
    return wall * 1e3 / steps, float(np.mean(durs)), float(np.min(durs))


def balance(pg, cfg, A, B, C, m, n, k, sched, gs=8, chunk=0):
    """Scheduler balance from one witness launch (after the timed steps): per
    program (one per CU at 256x256 tiles) the busy time from its start to its
    end, against the span of the whole launch."""
    import torch
    a = pg.make_args(tile=(256, 256, 64), group_size=gs, claim_chunk=chunk,
                     debug_flags=pg._abi.DEBUG_WITNESS)
    plan = pg.plan_gemm(cfg, m, n, k, "bf16_out_bf16", sched, a)
    G, T = plan["grid"], plan["tiles"]
    cfg.witness_enable(T, G)
    pg.pgemm_run(cfg, A, B, C, m, n, k, "bf16_out_bf16", sched, a)
    torch.cuda.synchronize()
    w = cfg.witness_read(T, G)
    us = 1e3 / cfg.info["wall_clock_khz"]               # microseconds per wall tick
    t0, t1 = w["t_start"][:G].astype(np.float64), w["t_end"][:G].astype(np.float64)
    busy = (t1 - t0) * us
    span = (t1.max() - t0.min()) * us
    tiles = w["n_tiles"][:G]
    X = cfg.info["num_xcds"]
    xcc = (w["hw_id"][:G].astype(np.int64) >> 16) & 0xF    # hardware XCC of each program
    q = np.arange(G)
    # programs that should share an XCD: workgroups go round robin over the
    # XCDs (from whichever XCD the hardware starts at), and program q is
    # workgroup q, or workgroup (q mod (G/X)) * X + q / (G/X) under XCD-major
    # numbering; share of programs on their group's most common XCD
    groups = q // (G // X) if plan["xcd_major"] else q % X
    together = sum(int(np.unique(xcc[groups == g], return_counts=True)[1].max()) for g in np.unique(groups))
    vals, counts = np.unique(tiles, return_counts=True)
    return {"span_us": round(span, 1), "busy_mean_us": round(float(busy.mean()), 1),
            "busy_min_us": round(float(busy.min()), 1), "busy_max_us": round(float(busy.max()), 1),
            "idle_frac": round(1.0 - float(busy.sum()) / (G * span), 4),
            "idle_frac_all_cus": round(1.0 - float(busy.sum()) / (cfg.info["num_cus"] * span), 4),
            "imbalance": round(float(busy.max() / busy.mean()), 4),
            "skew": round(float((busy.max() - busy.min()) / busy.mean()), 4),
            "programs": int(G),
            "tiles_min": int(tiles.min()), "tiles_max": int(tiles.max()),
            "tiles_per_program_hist": {str(int(v)): int(c) for v, c in zip(vals, counts)},
            "tiles_per_xcc": [int(tiles[xcc == x].sum()) for x in range(X)],
            "programs_per_xcc": [int((xcc == x).sum()) for x in range(X)],
            "xcd_major": bool(plan["xcd_major"]),
            "xcc_as_numbered": round(together / G, 4)}


def measured_clock(pg, cfg, A, B, C, key):
    """Engine clock (GHz) the headline launch runs at: one witness launch after
    the timed steps; median over programs of shader cycles / wall time."""
    import torch
    sched, gs = key.rsplit("_g", 1) if "_g" in key else (key, "8")
    gs = gs.split("_")[0]
    if sched == "stream_k":
        return None  # no witness on the stream-K path
    a = pg.make_args(tile=(256, 256, 64), group_size=int(gs), debug_flags=pg._abi.DEBUG_WITNESS)
    plan = pg.plan_gemm(cfg, M, N, K, "bf16_out_bf16", sched, a)
    G, T = plan["grid"], plan["tiles"]
    cfg.witness_enable(T, G)
    pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", sched, a)
    torch.cuda.synchronize()
    w = cfg.witness_read(T, G)
    dt = (w["t_end"] - w["t_start"]) / (cfg.info["wall_clock_khz"] * 1e3)
    ok = dt > 0
    return round(float(np.median(w["cycles"][ok] / dt[ok])) / 1e9, 3)


def measured_traffic(target):
    """Counter-derived memory bytes per launch of a profile target, or None if
    its kernel sources changed since the counters were taken."""
    import hashlib
    rec = TRAFFIC.get(target)
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, "tile_scheduling_persistent_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != rec["sha256_16"]:
        return None
    return rec["read_bytes"] + rec["write_bytes"]


def rooflines(flops, head, fp8, add, cfg1):
    """One roofline record per measured kernel: achieved algorithmic work per
    launch / mean HIP-event launch time, against the peak of its bound, with
    the counter-derived memory traffic per launch where it was measured."""
    out = [{"kernel": "gemm_bf16", "workload": f"bf16 8192^3, bf16 C, 256x256x64, {HEADLINE[0]} g{HEADLINE[1]}",
            "bound": "mfma", "achieved": round(flops / (head["event_ms_mean"] * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "traffic": measured_traffic("bf16_8192cube_work_stealing")}]
    fp8_traffic = {("8192x8192x8192_256x256", "work_stealing"): "fp8_8192cube_work_stealing",
                   ("256x28672x8192_128x256", "work_stealing"): "fp8_256x28672x8192_128x256_work_stealing",
                   ("256x28672x8192_128x256", "grouped"): "fp8_256x28672x8192_128x256_grouped"}
    for key, sched, bound in [("8192x8192x8192_256x256", "work_stealing", "mfma"),
                              ("256x28672x8192_128x256", "work_stealing", "hbm"),
                              ("256x28672x8192_128x256", "grouped", "hbm"),
                              ("256x28672x8192_128x128", "work_stealing", "hbm")]:
        r = fp8.get(key, {}).get(sched)
        if not r:
            continue
        shape, tile = key.split("_")
        if bound == "mfma":
            out.append({"kernel": "gemm_fp8", "workload": f"fp8 e4m3 {shape}, block scales, {tile}x128, {sched}",
                        "bound": "mfma", "achieved": r["tflops"], "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                        "traffic": measured_traffic(fp8_traffic.get((key, sched)))})
        else:
            out.append({"kernel": "gemm_fp8", "workload": f"fp8 e4m3 {shape}, block scales, {tile}x128, {sched}",
                        "bound": "hbm", "achieved": r["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "traffic": measured_traffic(fp8_traffic.get((key, sched)))})
    for key in ("128x128_blocked", "128x128_work_stealing", "32x16_blocked", "32x16_work_stealing"):
        if key in add:
            out.append({"kernel": "padd", "workload": f"fp32 add 8192x8192, {key.replace('_', ' tiles, ', 1)}",
                        "bound": "hbm", "achieved": round(add[key]["gbs"], 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "traffic": measured_traffic(f"add_8192sq_{key}")})
    if cfg1:
        out.append({"kernel": "gemm_bf16", "workload": cfg1["workload"], "bound": "launch",
                    "achieved": cfg1["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "traffic": None,
                    "note": "16 tiles on 16 of 256 CUs: the matrix-core peak is not reachable"})
    for r in out:
        r["frac"] = round(r["achieved"] / r["peak"], 4)
    return out


def cpu_baseline(a_bits, b_bits):
    """The oracle on a bounded sample: CPU_ROWS full rows of C (K = 8192)."""
    from oracle import gemm as og
    from oracle.codecs import bf16_to_f64
    rows = np.arange(CPU_ROWS) * (M // CPU_ROWS)
    A = bf16_to_f64(a_bits[rows])
    B = bf16_to_f64(b_bits)
    t0 = time.perf_counter()
    og.gemm_f64(A, B)
    dt = time.perf_counter() - t0
    flops = 2.0 * len(rows) * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": og.num_threads(),
            "kind": "oracle",
            "sample": f"{len(rows)} full rows of C ({len(rows)}x{N} outputs, K={K}; fp64 sum and |A||B| "
                      f"bound in one pass) in {dt:.2f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; --gpus must be 1 "
                                   "(the sharding plan is described, not run)"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.steps, args.warmup)
        return
    if args.profile_only:
        profile_only(args.profile_only, args.steps, args.warmup, args.settle)
        return
    import torch
    import tile_scheduling_persistent_amd as pg
    from synthetic import bf16_bits_normal, f32_normal

    cfg = pg.Config(0)
    stream = torch.cuda.current_stream()
    a_bits = bf16_bits_normal((M, K), 1030)
    b_bits = bf16_bits_normal((K, N), 1031)
    A = torch.from_numpy(a_bits.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    B = torch.from_numpy(b_bits.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    flops = 2.0 * M * N * K

    only = set(s for s in args.only.split(",") if s)
    settle(lambda: pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", HEADLINE[0],
                                pg.make_args(tile=(256, 256, 64), group_size=HEADLINE[1])), SETTLE_S)
    per = {}
    for sched, gs, chunk in SCHEDS:
        key = f"{sched}" + (f"_g{gs}" if sched != "blocked" and sched != "interleaved" else "") + \
            ("_pairs" if chunk < 0 else f"_c{chunk}" if chunk else "")
        if only and sched not in only and key not in only:
            continue
        a = pg.make_args(tile=(256, 256, 64), group_size=gs, claim_chunk=chunk)
        fn = lambda: pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", sched, a)  # noqa: E731
        ms, ev_mean, ev_min = time_calls(fn, args.steps, args.warmup, stream)
        per[key] = {"tflops": flops / (ms * 1e-3) / 1e12, "ms": ms, "event_ms_mean": ev_mean,
                    "event_ms_min": ev_min,
                    "frac_peak": flops / (ev_mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        print(f"# {key}: {ms:.4f} ms/step, {per[key]['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)

    # the two bf16 pipelines on the same workload (the default one is timed above)
    per_pipeline = {}
    if not args.skip_extra and not only:
        for pipe in ("four_wave", "pingpong"):
            row = {}
            for sched, gs, chunk in [("work_stealing", 8, 0), ("grouped", 8, 0), ("interleaved", 8, 0),
                                     ("blocked_grouped", 8, 0), ("work_stealing", 8, -1)]:
                a = pg.make_args(tile=(256, 256, 64), group_size=gs, claim_chunk=chunk, pipeline=pipe)
                fn = lambda: pg.pgemm_run(cfg, A, B, C, M, N, K, "bf16_out_bf16", sched, a)  # noqa: E731
                d = event_means(fn, args.steps, args.warmup, stream)
                row[sched + ("_pairs" if chunk < 0 else "")] = round(flops / (np.mean(d) * 1e-3) / 1e12, 2)
            per_pipeline[pipe] = row
            print(f"# 8192^3 {pipe}: {row}", file=sys.stderr, flush=True)

    # workload 1: 512^3 bf16, fp32 C, 128x128x64 tiles, blocked (16 tiles:
    # bound by launch and latency, not by the matrix cores)
    cfg1 = {}
    if not args.skip_extra:
        from synthetic import bf16_bits_uniform
        a1 = torch.from_numpy(bf16_bits_uniform((512, 512), 1010).view(np.int16)).to("cuda:0").view(torch.bfloat16)
        b1 = torch.from_numpy(bf16_bits_uniform((512, 512), 1011).view(np.int16)).to("cuda:0").view(torch.bfloat16)
        c1 = torch.empty((512, 512), dtype=torch.float32, device="cuda:0")
        args1 = pg.make_args(tile=(128, 128, 64))
        fn = lambda: pg.pgemm_run(cfg, a1, b1, c1, 512, 512, 512, "bf16_out_f32", "blocked", args1)  # noqa: E731
        d = event_means(fn, max(args.steps, 50), args.warmup, stream)
        gms = graph_ms_per_call(fn, 100, 5, stream)
        f1 = 2.0 * 512 ** 3
        cfg1 = {"workload": "bf16 512^3, fp32 C, 128x128x64 tiles, blocked (16 tiles)",
                "event_ms_mean": round(float(np.mean(d)), 5), "event_ms_median": round(float(np.median(d)), 5),
                "event_tflops": round(f1 / (np.mean(d) * 1e-3) / 1e12, 2),
                "graph_ms_per_call": round(gms, 5),
                "tflops": round(f1 / (gms * 1e-3) / 1e12, 2),
                "programs": pg.plan_gemm(cfg, 512, 512, 512, "bf16_out_f32", "blocked", args1)["grid"]}
        print(f"# cfg 1 (512^3): {cfg1}", file=sys.stderr, flush=True)

    # ragged, wave-quantised shapes (workload 4): every scheduler, in
    # RAGGED_ROUNDS interleaved rounds (each round times every scheduler once,
    # so clock drift spreads over all of them), at the default balanced grid
    # and at one program per CU (the pages' grid)
    ragged = {}
    if not args.skip_extra:
        from synthetic import bf16_bits_uniform
        ragged_scheds = [("blocked", 0), ("interleaved", 0), ("grouped", 0), ("blocked_grouped", 0),
                         ("work_stealing", 0), ("work_stealing_xcc", 0), ("work_stealing", -1),
                         ("work_stealing_xcc", -1), ("stream_k", 0)]
        static_keys = ["blocked", "interleaved", "grouped", "blocked_grouped"]
        ws_keys = ["work_stealing", "work_stealing_xcc", "work_stealing_pairs", "work_stealing_xcc_pairs"]
        for (m, n, k) in [(5120, 5120, 4096), (4864, 8000, 8192), (3000, 7000, 2048)]:
            ra = torch.from_numpy(bf16_bits_uniform((m, k), 1040 + m).view(np.int16)).to("cuda:0").view(torch.bfloat16)
            rb = torch.from_numpy(bf16_bits_uniform((k, n), 1041 + n).view(np.int16)).to("cuda:0").view(torch.bfloat16)
            rc = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
            f = 2.0 * m * n * k
            shape_rec = {}
            for grid_name, grid in [("balanced_grid", 0), ("grid_per_cu", cfg.info["num_cus"])]:
                calls = {}
                for sched, chunk in ragged_scheds:
                    if sched == "stream_k" and grid:
                        continue
                    a = pg.make_args(tile=(256, 256, 64), claim_chunk=chunk, grid=grid)
                    calls[sched + ("_pairs" if chunk < 0 else "")] = (
                        lambda a=a, sched=sched: pg.pgemm_run(cfg, ra, rb, rc, m, n, k, "bf16_out_bf16", sched, a))
                settle(next(iter(calls.values())), 0.5)
                means = {key: [] for key in calls}
                for _ in range(RAGGED_ROUNDS):
                    for key, fn in calls.items():
                        means[key].append(float(np.mean(event_means(fn, args.steps, 3, stream))))
                rec = {key: rounds_summary(f, v) for key, v in means.items()}
                best_static = max(static_keys, key=lambda x: rec[x]["median"])
                best_ws = max(ws_keys, key=lambda x: rec[x]["median"])
                rec["_summary"] = {
                    "programs": pg.plan_gemm(cfg, m, n, k, "bf16_out_bf16", "work_stealing",
                                             pg.make_args(tile=(256, 256, 64), grid=grid))["grid"],
                    "best_static": best_static, "best_work_stealing": best_ws,
                    "work_stealing_over_best_static": round(rec["work_stealing"]["median"]
                                                            / rec[best_static]["median"], 4),
                    "best_work_stealing_over_best_static": round(rec[best_ws]["median"]
                                                                 / rec[best_static]["median"], 4)}
                shape_rec[grid_name] = rec
                print(f"# ragged {m}x{n}x{k} {grid_name}: " +
                      ", ".join(f"{s_}={v['median']}" for s_, v in rec.items() if not s_.startswith("_")) +
                      f"; {rec['_summary']}", file=sys.stderr, flush=True)
            ragged[f"{m}x{n}x{k}"] = shape_rec
            del ra, rb, rc

    # under-filled shapes (fewer 256x256 tiles than CUs, e.g. one GPU's share
    # of an 8-way split of 8192^3): stream-K against the data-parallel
    # schedulers, and against smaller tiles as the other way to fill the chip
    skinny = {}
    if not args.skip_extra:
        from synthetic import bf16_bits_uniform
        for (m, n, k) in [(8192, 1024, 8192), (1024, 8192, 8192), (2048, 2048, 8192)]:
            ra = torch.from_numpy(bf16_bits_uniform((m, k), 1060 + m).view(np.int16)).to("cuda:0").view(torch.bfloat16)
            rb = torch.from_numpy(bf16_bits_uniform((k, n), 1061 + n).view(np.int16)).to("cuda:0").view(torch.bfloat16)
            rc = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
            f = 2.0 * m * n * k
            row = {}
            for sched, tile in [("grouped", (256, 256, 64)), ("work_stealing", (256, 256, 64)),
                                ("stream_k", (256, 256, 64)), ("grouped", (128, 128, 64)),
                                ("work_stealing", (128, 128, 64)), ("stream_k", (128, 128, 64))]:
                a = pg.make_args(tile=tile)
                fn = lambda: pg.pgemm_run(cfg, ra, rb, rc, m, n, k, "bf16_out_bf16", sched, a)  # noqa: E731
                _, ev_mean, _ = time_calls(fn, args.steps, args.warmup, stream)
                row[f"{sched}_{tile[0]}"] = {"tflops": round(f / (ev_mean * 1e-3) / 1e12, 2),
                                             "event_ms_mean": round(ev_mean, 5)}
            skinny[f"{m}x{n}x{k}"] = row
            print(f"# skinny {m}x{n}x{k}: " + ", ".join(f"{s_}={v['tflops']}" for s_, v in row.items()),
                  file=sys.stderr, flush=True)
            del ra, rb, rc

    # one slow XCD (every program on hardware XCC 0 waits 50 us before each
    # tile, about one tile's time; a stand-in for an XCD shared with other
    # work): per-XCD work stealing against stealing across XCDs, 8192x8192x2048
    slow_xcc = {}
    if not args.skip_extra and (not only or "work_stealing_xcc_g8" in only):
        k2 = 2048
        sa = torch.from_numpy(bf16_bits_normal((M, k2), 1070).view(np.int16)).to("cuda:0").view(torch.bfloat16)
        sb = torch.from_numpy(bf16_bits_normal((k2, N), 1071).view(np.int16)).to("cuda:0").view(torch.bfloat16)
        f = 2.0 * M * N * k2
        for slow in (False, True):
            for sched in ["grouped", "work_stealing", "work_stealing_xcc"]:
                a = pg.make_args(tile=(256, 256, 64),
                                 debug_flags=pg._abi.DEBUG_STRAGGLER_XCC if slow else 0,
                                 straggler_program=0 if slow else -1, straggler_ns=50_000 if slow else 0)
                fn = lambda: pg.pgemm_run(cfg, sa, sb, C, M, N, k2, "bf16_out_bf16", sched, a)  # noqa: E731
                _, ev_mean, _ = time_calls(fn, args.steps, args.warmup, stream)
                slow_xcc[f"{sched}{'_slow' if slow else ''}"] = {
                    "tflops": round(f / (ev_mean * 1e-3) / 1e12, 2), "event_ms_mean": round(ev_mean, 5)}
        print(f"# 8192x8192x2048, XCC 0 slowed by 50 us per tile: {slow_xcc}", file=sys.stderr, flush=True)
        del sa, sb

    # several GEMMs in one persistent launch (experts of different sizes)
    # against one launch per GEMM
    grouped_gemm = {}
    if not args.skip_extra:
        from synthetic import bf16_bits_uniform
        ms = [512, 1024, 256, 768, 2048, 128, 1536, 640]
        gn, gk = 2048, 4096
        probs = []
        for g, m in enumerate(ms):
            ga = torch.from_numpy(bf16_bits_uniform((m, gk), 1080 + g).view(np.int16)).to("cuda:0").view(torch.bfloat16)
            gb = torch.from_numpy(bf16_bits_uniform((gk, gn), 1090 + g).view(np.int16)).to("cuda:0").view(torch.bfloat16)
            probs.append((ga, gb, torch.empty((m, gn), dtype=torch.bfloat16, device="cuda:0"), m, gn, gk))
        f = sum(2.0 * m * gn * gk for m in ms)
        for sched in ["grouped", "work_stealing"]:
            for tile in [(256, 256, 64), (128, 128, 64)]:
                a = pg.make_args(tile=tile)
                fn = lambda: pg.pgemm_run_grouped(cfg, probs, "bf16_out_bf16", sched, a)  # noqa: E731
                _, ev_one, _ = time_calls(fn, args.steps, args.warmup, stream)

                def separate():
                    for pr in probs:
                        pg.pgemm_run(cfg, *pr, "bf16_out_bf16", sched, a)
                _, ev_sep, _ = time_calls(separate, args.steps, args.warmup, stream)
                grouped_gemm[f"{sched}_{tile[0]}"] = {
                    "one_launch_tflops": round(f / (ev_one * 1e-3) / 1e12, 2),
                    "one_launch_per_gemm_tflops": round(f / (ev_sep * 1e-3) / 1e12, 2)}
        # the same experts in block-scaled fp8 (256x256x128 tiles)
        from synthetic import fp8_blockscaled
        fprobs = []
        for g, m in enumerate(ms):
            qa, sa = fp8_blockscaled(m, gk, 1100 + g, 1120 + g, k_major=True)
            qb, sb = fp8_blockscaled(gn, gk, 1110 + g, 1130 + g, k_major=False)
            fprobs.append((torch.from_numpy(qa).to("cuda:0"), torch.from_numpy(qb).to("cuda:0"),
                           torch.empty((m, gn), dtype=torch.bfloat16, device="cuda:0"), m, gn, gk,
                           torch.from_numpy(sa).to("cuda:0"), torch.from_numpy(sb).to("cuda:0")))
        for sched in ["grouped", "work_stealing"]:
            fn = lambda: pg.pgemm_run_grouped(cfg, fprobs, "fp8_b128_out_bf16", sched)  # noqa: E731
            _, ev_one, _ = time_calls(fn, args.steps, args.warmup, stream)

            def separate_fp8():
                for pr in fprobs:
                    pg.pgemm_run(cfg, *pr[:6], "fp8_b128_out_bf16", sched,
                                 pg.make_args(a_scale=pr[6], b_scale=pr[7]))
            _, ev_sep, _ = time_calls(separate_fp8, args.steps, args.warmup, stream)
            grouped_gemm[f"fp8_{sched}_256"] = {
                "one_launch_tflops": round(f / (ev_one * 1e-3) / 1e12, 2),
                "one_launch_per_gemm_tflops": round(f / (ev_sep * 1e-3) / 1e12, 2)}
        print(f"# grouped GEMM ({len(ms)} problems, M = {ms}, N={gn}, K={gk}): {grouped_gemm}",
              file=sys.stderr, flush=True)
        del probs, fprobs

    # per-CU busy / idle skew of each scheduler (witness launches, untimed):
    # 8192^3 and the ragged shapes
    bal = {}
    if not args.skip_extra:
        from synthetic import bf16_bits_uniform
        scheds = [("blocked", 8, 0), ("interleaved", 8, 0), ("grouped", 8, 0), ("blocked_grouped", 8, 0),
                  ("work_stealing", 8, 0), ("work_stealing_xcc", 8, 0), ("work_stealing", 8, -1)]
        shapes = [(M, N, K, A, B, C)]
        for (m, n, k) in [(5120, 5120, 4096), (4864, 8000, 8192), (3000, 7000, 2048)]:
            ra = torch.from_numpy(bf16_bits_uniform((m, k), 1040 + m).view(np.int16)).to("cuda:0").view(torch.bfloat16)
            rb = torch.from_numpy(bf16_bits_uniform((k, n), 1041 + n).view(np.int16)).to("cuda:0").view(torch.bfloat16)
            shapes.append((m, n, k, ra, rb, torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")))
        for (m, n, k, ta, tb, tc) in shapes:
            row = {}
            for sched, gs, chunk in scheds:
                row[sched + ("_pairs" if chunk < 0 else "")] = balance(pg, cfg, ta, tb, tc, m, n, k, sched, gs, chunk)
            bal[f"{m}x{n}x{k}"] = row
            print(f"# balance {m}x{n}x{k}: " + ", ".join(f"{s_}: idle {v['idle_frac']} skew {v['skew']}"
                                                         for s_, v in row.items()), file=sys.stderr, flush=True)
            ws = row["work_stealing"]
            print(f"#   {ws['programs']} programs, on the XCC of their p mod X class: {ws['xcc_as_numbered']:.0%}; "
                  f"work stealing tiles per XCC {ws['tiles_per_xcc']}, per program {ws['tiles_per_program_hist']}",
                  file=sys.stderr, flush=True)
        del shapes

    # block-scaled fp8 (workload 5): work stealing vs grouped
    fp8 = {}
    if not args.skip_extra:
        from synthetic import fp8_blockscaled
        for (m, n, k, tile) in [(256, 28672, 8192, (128, 128, 128)), (256, 28672, 8192, (128, 256, 128)),
                                (256, 28672, 8192, (256, 256, 128)), (8192, 8192, 8192, (256, 256, 128))]:
            qa, sa = fp8_blockscaled(m, k, 1050, 1052, k_major=True)
            qb, sb = fp8_blockscaled(n, k, 1051, 1053, k_major=False)
            dA, dB = torch.from_numpy(qa).to("cuda:0"), torch.from_numpy(qb).to("cuda:0")
            dSA, dSB = torch.from_numpy(sa).to("cuda:0"), torch.from_numpy(sb).to("cuda:0")
            dC = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
            f = 2.0 * m * n * k
            nbytes = m * k + k * n + (m + n) * (k // 128) + 2 * m * n
            # interleaved rounds of the schedulers, each batch right after that
            # scheduler's own settle (the clock under one kernel's sustained
            # load differs from another's)
            calls = {}
            for sched in ["grouped", "work_stealing", "stream_k"]:
                a = pg.make_args(tile=tile, a_scale=dSA, b_scale=dSB)
                calls[sched] = (a, lambda a=a, sched=sched: pg.pgemm_run(cfg, dA, dB, dC, m, n, k,
                                                                         "fp8_b128_out_bf16", sched, a))
            means = {s_: [] for s_ in calls}
            for _ in range(RAGGED_ROUNDS):
                for s_, (_, fn) in calls.items():
                    settle(fn, ROOFLINE_SETTLE_S)
                    means[s_].append(event_batch_ms(fn, args.steps, 3, stream))
            row = {}
            for sched, (a, _) in calls.items():
                ev_mean = float(np.median(means[sched]))
                plan = pg.plan_gemm(cfg, m, n, k, "fp8_b128_out_bf16", sched, a)
                row[sched] = {"tflops": round(f / (ev_mean * 1e-3) / 1e12, 2),
                              "gbs": round(nbytes / (ev_mean * 1e-3) / 1e9, 1),
                              "batch_ms_per_call": round(ev_mean, 5),
                              "rounds_gbs": rounds_summary(nbytes, means[sched], 1e9),
                              "grid": plan["grid"], "xcd_major": plan["xcd_major"]}
            fp8[f"{m}x{n}x{k}_{tile[0]}x{tile[1]}"] = row
            print(f"# fp8 {m}x{n}x{k}: {row}", file=sys.stderr, flush=True)
            del dA, dB, dC, qa, qb

    add = {}
    if not args.skip_add:
        R = Cc = 8192
        X = torch.from_numpy(f32_normal((R, Cc), 2001)).to("cuda:0")
        Y = torch.from_numpy(f32_normal((R, Cc), 2002)).to("cuda:0")
        Z = torch.empty_like(X)
        nbytes = 3 * R * Cc * 4
        for tile in [(32, 16), (128, 128)]:
            for sched in ["blocked", "interleaved", "grouped", "work_stealing"]:
                fn = lambda: pg.padd_run(cfg, X, Y, Z, R, Cc, tile[0], tile[1], sched)  # noqa: E731
                settle(fn, 3 * ROOFLINE_SETTLE_S)
                ev_mean = float(np.median([event_batch_ms(fn, max(args.steps, 20), 2, stream)
                                           for _ in range(RAGGED_ROUNDS)]))
                add[f"{tile[0]}x{tile[1]}_{sched}"] = {"gbs": nbytes / (ev_mean * 1e-3) / 1e9,
                                                       "batch_ms_per_call": ev_mean}
                print(f"# add {tile} {sched}: {nbytes / (ev_mean * 1e-3) / 1e9:.0f} GB/s",
                      file=sys.stderr, flush=True)

    # the same workloads through torch's own kernels on this GPU (context,
    # not a baseline): hipBLASLt for the 8192^3 bf16 GEMM, torch.add
    vendor = {}
    if not args.skip_extra:
        Ct = torch.empty_like(C)
        fn = lambda: torch.matmul(A, B, out=Ct)  # noqa: E731
        _, ev_mean, _ = time_calls(fn, args.steps, args.warmup, stream)
        vendor["torch_matmul_bf16_8192cube_tflops"] = round(flops / (ev_mean * 1e-3) / 1e12, 2)
        del Ct
    if not args.skip_add:
        fn = lambda: torch.add(X, Y, out=Z)  # noqa: E731
        _, ev_mean, _ = time_calls(fn, max(args.steps, 20), args.warmup, stream)
        vendor["torch_add_8192sq_gbs"] = round(3 * 8192 * 8192 * 4 / (ev_mean * 1e-3) / 1e9, 1)
    if vendor:
        print(f"# torch on the same workloads: {vendor}", file=sys.stderr, flush=True)

    # several adds in one persistent launch against one launch per add
    multi_add = {}
    if not args.skip_add:
        shapes = [(4096, 4096), (2048, 8192), (8192, 1024), (1000, 3000), (513, 700)]
        ops = []
        for g, (r, c) in enumerate(shapes):
            x = torch.from_numpy(f32_normal((r, c), 2100 + 2 * g)).to("cuda:0")
            y = torch.from_numpy(f32_normal((r, c), 2101 + 2 * g)).to("cuda:0")
            ops.append((x, y, torch.empty_like(x), r, c))
        nbytes = sum(3 * r * c * 4 for r, c in shapes)
        for tile in [(32, 16), (128, 128)]:
            for sched in ["blocked", "work_stealing"]:
                fn = lambda: pg.padd_run_multi(cfg, ops, tile[0], tile[1], sched)  # noqa: E731
                _, ev_multi, _ = time_calls(fn, max(args.steps, 20), args.warmup, stream)

                def separate():
                    for o in ops:
                        pg.padd_run(cfg, *o, tile[0], tile[1], sched)
                _, ev_sep, _ = time_calls(separate, max(args.steps, 20), args.warmup, stream)
                multi_add[f"{tile[0]}x{tile[1]}_{sched}"] = {
                    "one_launch_gbs": round(nbytes / (ev_multi * 1e-3) / 1e9, 1),
                    "one_launch_per_add_gbs": round(nbytes / (ev_sep * 1e-3) / 1e9, 1)}
        print(f"# several adds ({len(shapes)} problems): {multi_add}", file=sys.stderr, flush=True)
        del ops

    head_key = f"{HEADLINE[0]}_g{HEADLINE[1]}"
    if head_key not in per:
        head_key = next(iter(per))
    h = per[head_key]
    clock_ghz = measured_clock(pg, cfg, A, B, C, head_key)
    head_plan = pg.plan_gemm(cfg, M, N, K, "bf16_out_bf16", head_key.rsplit("_g", 1)[0],
                             pg.make_args(tile=(256, 256, 64)))
    line = {
        "metric": "GEMM TFLOP/s & % MFMA peak per scheduler (8192^3 bf16); add GB/s",
        "value": round(h["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: A, B iid normal(0,1) rounded to bf16 (PCG64 seeds 1030/1031)",
        "config": {"workload": "bf16 GEMM M=N=K=8192, fp32 accumulate, bf16 C, 256x256x64 tiles, "
                               f"persistent grid = {head_plan['grid']} programs ({cfg.info['num_cus']} CUs x "
                               f"{head_plan['occupancy']}), scheduler {head_key}",
                   "M": M, "N": N, "K": K, "scheduler": head_key},
        "roofline": {"bound": "mfma", "achieved": round(flops / (h["event_ms_mean"] * 1e-3) / 1e12, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (h["event_ms_mean"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("bf16_8192cube_work_stealing"),
                     "clock_ghz_measured": clock_ghz,
                     "peak_at_measured_clock": (round(PEAK_BF16_TFLOPS * clock_ghz / PEAK_CLOCK_GHZ, 1)
                                                if clock_ghz else None),
                     "frac_at_measured_clock": (round(flops / (h["event_ms_mean"] * 1e-3) / 1e12
                                                      / (PEAK_BF16_TFLOPS * clock_ghz / PEAK_CLOCK_GHZ), 4)
                                                if clock_ghz else None),
                     "traffic_unit": "bytes per launch the L2s send to the memory controllers (Infinity Cache hits included)",
                     "algorithmic_bytes": 2 * (M * K + K * N + M * N)},
        "rooflines": rooflines(flops, h, fp8, add, cfg1),
        "per_scheduler": {k: {"tflops": round(v["tflops"], 2), "frac_peak": round(v["frac_peak"], 4),
                              "event_ms_mean": round(v["event_ms_mean"], 5)} for k, v in per.items()},
        "per_pipeline": per_pipeline,
        "default_pipeline": head_plan["kernel"],
        "cfg1_512cube": cfg1,
        "add": {k: {"gbs": round(v["gbs"], 1), "frac_hbm": round(v["gbs"] / PEAK_HBM_GBS, 4)}
                for k, v in add.items()},
        "ragged": ragged,
        "multi_add": multi_add,
        "grouped_gemm": grouped_gemm,
        "skinny": skinny,
        "slow_xcc": slow_xcc,
        "fp8": fp8,
        "balance": bal,
        "torch_same_box": vendor,
        "device": cfg.info,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(a_bits, b_bits)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the all-reduce hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload grad7b]
                    [--mode fused|stepwise|graph|tree|tree_stepwise]
                    [--collective all_reduce|reduce_scatter|all_gather|all_to_all]
                    [--op OP] [--multi] [--access auto|streaming|cached] [--no-cpu-baseline]
    python bench.py --sweep            # 1 KiB..256 MiB per rank, every mode, alpha-beta fit
    python bench.py --copy-probe BYTES # a plain device copy (HBM counter calibration)

One "step" is one call of the collective on the whole workload: every
virtual rank's buffer (inputs already resident in HBM) reduced and the result
written back to every rank. The default workload is the 7e9-element fp16
gradient per rank (14 GB, the 7B model of the geek-doc page "训练梯度同步与
集合通信", sections 一 and 四) at 8 virtual ranks, AVG with fp32
accumulation, fused mode, in place. The rank buffers are allocated and timed
twice; the second pass is reported (the first as
first_allocation_ms_per_step). Calls whose rank buffers fit in the
last-level cache rotate buffer sets so every timed call reads HBM.

Reported (one JSON line):
  value        algbw = S / T, S = bytes per rank (handbook "集合通信原语",
               section 算法带宽与总线带宽)
  busbw        algbw * 2(N-1)/N for all-reduce, (N-1)/N for the others
               (same section)
  ms_per_step  the K timed steps between two events, over K
  step_ms      median / min / max of single steps, from a second pass of K
               steps with an event after each
  roofline     the call's algorithmic HBM bytes (all-reduce and all-to-all
               2*N*S, reduce-scatter and all-gather (N+1)*S) over its time,
               against the 8 TB/s HBM peak; traffic = bytes the HBM counters
               saw per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a
               plain copy's reading; one launch in fused mode, the sum of the
               2(N-1) launches in stepwise mode), from the committed profile
               of that workload, mode and collective when it matches the
               current kernel source, else null
  moved        stepwise and graph modes: the bytes the ring's steps move
               (5(N-1)*S for fp32/int32, (14N-18)*count with the fp32
               workspace of fp16/bf16) and their rate
  copy_ceiling a plain 1 GiB device copy timed in the same process: the
               practical read-once write-once rate of this machine, and the
               call's rate over it
  same_buffer_copy (all-reduce) a plain copy of each rank buffer into the
               next one, on the call's own allocations: the same bytes as the
               call, and the call's rate over it
  cpu_baseline the CPU oracle on the workload, or a window of it, in the same
               unit: the literal ring on the host's threads (OMP_NUM_THREADS,
               else the affinity mask), and beside it the per-element fold
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "all-reduce algbw/busbw GB/s and % HBM peak, N=8 ranks, 64 MiB–14 GB msgs"
HBM_PEAK_GBPS = 8000.0
LLC_BYTES = 256 << 20      # MI355X last-level (Infinity) cache
ROTATE_BYTES = 1 << 30    # rotated footprint for calls that fit in it
COPY_CEILING_BYTES = 1 << 30  # plain copy timed beside every bench line
CSRC = os.path.join(ROOT, "ring_all_reduce_ar_amd", "csrc")

# workload name -> (nranks, count, dtype, op, description)
WORKLOADS = {
    "small": (4, 4096, "f32", "sum",
              "small: 4 virtual ranks x 4096 fp32, uniform[-1,1), SUM, in place (the handbook's 4-rank ring shape)"),
    "grad7b": (8, 7_000_000_000, "f16", "avg",
               "grad7b: 8 virtual ranks x 7e9 fp16 gradient (14 GB per rank), N(0,1e-3^2) with 1% N(0,1) "
               "outliers, AVG with fp32 accumulation, in place"),
    "bucket25": (8, 6_553_600, "f32", "avg",
                 "bucket25: 8 virtual ranks x one 25 MiB fp32 DDP bucket, N(0,1e-3^2), AVG, in place"),
    "sweep64m": (8, 16_777_216, "f32", "sum", "sweep point: 8 virtual ranks x 64 MiB fp32, uniform[-1,1), SUM, in place"),
    "sweep256m": (8, 67_108_864, "f32", "sum",
                  "sweep point: 8 virtual ranks x 256 MiB fp32, uniform[-1,1), SUM, in place"),
    "bucket64": (64, 67_108_864, "f32", "max",
                 "bucket64: 64 virtual ranks x 256 MiB fp32 bucket, uniform[-1,1), MAX, in place"),
    "bucket8": (8, 67_108_864, "f32", "max",
                "bucket8: 8 virtual ranks x 256 MiB fp32 bucket, uniform[-1,1), MAX, in place"),
}
ESIZE = {"f32": 4, "f16": 2, "bf16": 2, "i32": 4}
CPU_WINDOW_LOG2 = 27  # elements per rank in the CPU oracle's window (about 10 s of oracle work)
CPU_MIN_SECONDS = 5.0  # a shorter sample is repeated until this much oracle time has passed


def alpha_beta_time(nranks: int, msg_bytes: float, alpha_s: float, beta_bytes_per_s: float):
    """Ring all-reduce time in the alpha-beta model (geek-doc page "训练梯度同步
    与集合通信", section 四; handbook "集合通信原语", section α-β 模型):
    T = 2(N-1)*alpha + 2(N-1)/N * M / beta. Returns (latency term, bandwidth
    term, total) in seconds."""
    lat = 2 * (nranks - 1) * alpha_s
    bw = 2 * (nranks - 1) / nranks * msg_bytes / beta_bytes_per_s
    return lat, bw, lat + bw


def ring_moved_bytes(nranks: int, count: int, dtype: str) -> int:
    """HBM bytes one stepwise ring all-reduce moves, summed over its 2(N-1)
    launches (the ring of the geek-doc page "训练梯度同步与集合通信", section
    三). Every step touches each element once, at one rank or another.
    fp32/int32 partials travel in the rank buffers: a reduce-scatter step
    reads 2e and writes e bytes per element, an all-gather step reads e and
    writes e, so 5(N-1)*count*e in all. fp16/bf16 partials stay in an fp32
    workspace: the first reduce-scatter step reads 2+2 and writes 4 bytes,
    a middle step reads 2+4 and writes 4, the last reads 2+4 and writes 2
    (at N = 2 the one step reads 2+2 and writes 2), and an all-gather step
    reads 2 and writes 2: (14N-18)*count in all."""
    if nranks < 2:
        return 0
    if dtype in ("f16", "bf16"):
        return (14 * nranks - 18) * count
    return 5 * (nranks - 1) * count * ESIZE[dtype]


def fit_line(xs, ys):
    """Least-squares y = a + b*x; returns (a, b)."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    b = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sxx if sxx else 0.0
    return my - b * mx, b


SWEEP_LATENCY_MAX = 1 << 20  # bytes per rank: the latency regime of the sweep


def alpha_beta_fit(points, launches: int, nranks: int):
    """The alpha-beta model T = launches*alpha + moved/beta fitted in the two
    regimes where each term shows: alpha from the intercept of a line through
    the calls of at most SWEEP_LATENCY_MAX bytes per rank, beta from the
    slope of a line through the calls whose in-place footprint N*S exceeds
    the last-level cache (HBM-bound). Sizes in between run from that cache
    and would pull a single line's slope up and its intercept down.
    points: (bytes per rank, moved bytes, seconds). Returns (alpha seconds
    per launch, beta bytes per second or None)."""
    lat = [(m, t) for s, m, t in points if s <= SWEEP_LATENCY_MAX]
    hbm = [(m, t) for s, m, t in points if nranks * s > LLC_BYTES]
    a, _ = fit_line(*zip(*lat))
    b = fit_line(*zip(*hbm))[1] if len(hbm) >= 2 else 0.0
    return a / launches, (1.0 / b if b > 0 else None)


def kernel_sha() -> str:
    """Hash of every kernel source and of the launch code (grid shapes):
    counters taken on other sources are not reported."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, mode: str, collective: str = "all_reduce"):
    """Per-launch HBM bytes from the committed counter summary, if it was taken
    on the current kernel source; else None. All-reduce summaries are
    traffic_<workload>_<mode>.md, the other collectives'
    traffic_<workload>_<mode>_<collective>.md."""
    suffix = "" if collective == "all_reduce" else f"_{collective}"
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{mode}{suffix}.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    m = re.search(r"kernel_sha:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_sha():
        return None
    return float(t.group(1))


def cpu_threads() -> int:
    """Host threads for the CPU oracle: OMP_NUM_THREADS when set (the host's
    CPU share for this job), else every core in this process's affinity mask."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    t = int(env) if env.isdigit() and int(env) > 0 else len(os.sched_getaffinity(0))
    return max(1, min(t, 256))


def _time_repeated(fn, min_seconds):
    """Calls fn until min_seconds have passed; returns (calls, seconds)."""
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            return reps, dt


def cpu_baseline(nranks: int, dtype: str, op: str, workload: str, coll: str = "all_reduce", count: int = 0):
    """The oracle on a sample of the same workload, timed on the host's cores.
    All-reduce: the literal ring with every ring half-step split over
    (rank x piece) on T threads and a barrier between half-steps (the ranks
    of the handbook's ring step together: "集合通信原语", section 环形 all-reduce
    与通信量) is `value`; the per-element fold on the same T threads is timed
    beside it (`fold`). The other collectives run the oracle's serial
    reduce-scatter, all-gather or all-to-all on one thread. The sample is the
    workload itself when its `count` elements per rank fit in
    2^CPU_WINDOW_LOG2, else a window of that many elements per rank, seeded
    the same way; a sample that runs in under CPU_MIN_SECONDS is repeated
    until that much time has passed. algbw convention as the GPU line."""
    import oracle
    import synthetic
    window = 1 << CPU_WINDOW_LOG2
    sample = min(count, window) if count > 0 else window
    wl = workload if workload in synthetic.WORKLOAD_IDS else "sweep"
    in_count = sample // nranks if coll == "all_gather" else sample
    # generated on the device (fast), copied to host memory before timing
    import torch
    dev = "cuda" if torch.cuda.is_available() else "cpu"
    xs = [synthetic.to_numpy(t) for t in synthetic.rank_inputs(wl, nranks, in_count, dtype, device=dev, op=op)]
    threads = cpu_threads() if coll == "all_reduce" else 1
    what = {"all_reduce": f"literal ring (N-1 reduce-scatter + N-1 all-gather steps, each half-step over "
                          f"rank x piece on {threads} threads, a barrier between half-steps)",
            "reduce_scatter": "reduce-scatter, single thread", "all_gather": "all-gather, single thread"}.get(
        coll, "all-to-all, single thread")
    if coll == "all_reduce":
        bufs = [a.copy() for a in xs]
        reps, dt = _time_repeated(lambda: oracle.ring_all_reduce_threads(bufs, dtype, op, threads), CPU_MIN_SECONDS)
        outs = [np.empty_like(a) for a in xs]
        freps, fdt = _time_repeated(lambda: oracle.fold_all_reduce_threads(xs, dtype, op, threads, out=outs),
                                    CPU_MIN_SECONDS)
        del bufs, outs
    else:
        fn = {"reduce_scatter": lambda: oracle.reduce_scatter(xs, dtype, op),
              "all_gather": lambda: oracle.all_gather(xs, dtype)}.get(coll, lambda: oracle.all_to_all(xs, dtype))
        reps, dt = _time_repeated(fn, CPU_MIN_SECONDS)
    s_bytes = sample * ESIZE[dtype]
    part = "the whole workload" if sample == count else f"a window of the {count}-element workload" if count else "a window"
    out = {"value": s_bytes * reps / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{nranks} ranks x {sample} {dtype} elements per rank ({s_bytes / 2**20:.1f} MiB; {part}), "
                     f"{what}, {op}" + (f", {reps} calls" if reps > 1 else ""),
           "seconds": dt}
    if coll == "all_reduce":
        out["fold"] = {"value": s_bytes * freps / fdt / 1e9, "unit": "GB/s", "cores": threads, "seconds": fdt,
                       "calls": freps,
                       "form": "per-element fold (acc = x_c[i]; acc = x_{c+k}[i] (+) acc), contiguous element "
                               "ranges on the same threads"}
    return out


def sig(x: float, digits: int = 6) -> float:
    """x rounded to `digits` significant digits (the line's rates span
    0.001 to 10^4 GB/s)."""
    return float(f"{x:.{digits}g}")


def time_steps(torch, stream, step, k: int, warmup: int, rotate: bool = True, per_step_events: bool = False):
    """Warm up, then time exactly k calls of step(i) on `stream`. The timed
    pass brackets the k calls with two events only: an event recorded between
    kernels costs the stream a few microseconds, which shows at short calls.
    With per_step_events an event follows every call instead. Returns
    (ms per call, None) or (None, [ms of each call])."""
    for i in range(warmup):
        step(i if rotate else 0)
    torch.cuda.synchronize()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1 if per_step_events else 2)]
    torch.cuda.synchronize()
    events[0].record(stream)
    for i in range(k):
        step(i if rotate else 0)
        if per_step_events:
            events[i + 1].record(stream)
    if not per_step_events:
        events[1].record(stream)
    torch.cuda.synchronize()
    if not per_step_events:
        return events[0].elapsed_time(events[1]) / k, None
    return None, [events[i].elapsed_time(events[i + 1]) for i in range(k)]


# The metric's range at 8 ranks below the headline size, timed after it in
# the default run: (workload, steps). Each point allocates its rank buffers
# twice and reports the second allocation (the first beside it), as the
# headline does; bucket25 rotates buffer sets so every call reads HBM.
RANGE_POINTS = (("sweep64m", 100), ("sweep256m", 50), ("bucket25", 200))


def range_point(torch, ar, synthetic, name: str, steps: int, warmup: int, copy_gbps: float):
    """One fused in-place all-reduce workload of the metric's range, timed as
    the headline is (two allocations, rotation below the last-level cache)."""
    n, count, dtype, op, desc = WORKLOADS[name]
    wl = name if name in synthetic.WORKLOAD_IDS else "sweep"
    s_bytes = count * ESIZE[dtype]
    sets = 1 if n * s_bytes > LLC_BYTES else -(-ROTATE_BYTES // (n * s_bytes))
    stream = torch.cuda.current_stream()
    times = []
    with ar.Comm(n, 0) as comm:
        for _ in range(2):
            bufsets = [synthetic.rank_inputs(wl, n, count, dtype, device="cuda", op=op, salt=k) for k in range(sets)]
            ptrsets = [[b.data_ptr() for b in bufs] for bufs in bufsets]

            def step(i):
                p = ptrsets[i % sets]
                ar.ar_all_reduce(comm, p, p, count, dtype, op, "fused", stream)

            times.append(time_steps(torch, stream, step, steps, warmup)[0])
            sb_ms = same_buffer_copy_ms(torch, ar, ptrsets[0], s_bytes, stream) if s_bytes % 16 == 0 else None
            del bufsets, ptrsets
            torch.cuda.empty_cache()
    ms = times[1]
    alg = 2 * n * s_bytes / (ms * 1e-3) / 1e9
    algbw = s_bytes / (ms * 1e-3) / 1e9
    return {"workload": desc, "nranks": n, "bytes_per_rank": s_bytes, "dtype": dtype, "op": op, "mode": "fused",
            "steps": steps, "rotating_buffer_sets": sets, "ms_per_step": sig(ms),
            "first_allocation_ms_per_step": sig(times[0]), "algbw_gbps": sig(algbw),
            "busbw_gbps": sig(algbw * 2 * (n - 1) / n), "hbm_gbps": sig(alg),
            "hbm_frac": sig(alg / HBM_PEAK_GBPS), "achieved_over_copy": sig(alg / copy_gbps),
            "same_buffer_copy": None if sb_ms is None else {
                "ms": sig(sb_ms), "hbm_frac": sig(2 * n * s_bytes / (sb_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS),
                "achieved_over_copy": sig(sb_ms / ms)}}


def same_buffer_copy_ms(torch, ar, ptrs, nbytes: int, stream, steps: int = 5):
    """A plain copy on the call's own rank buffers: rank r's buffer into rank
    r+1's, for every r (one-rank all-gathers, 16-byte vectors), so every
    buffer is read once and written once, 2*N*nbytes in all, the all-reduce's
    bytes on the same allocations. Overwrites the buffers. Returns ms per
    pass over the N buffers (best of `steps`)."""
    n = len(ptrs)
    best = None
    with ar.Comm(1, 0) as comm:
        def one():
            for r in range(n):
                ar.ar_all_gather(comm, [ptrs[r]], [ptrs[(r + 1) % n]], nbytes // 4, "i32", "fused", stream)
        one()
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            one()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1)
            best = t if best is None else min(best, t)
    return best


def time_copy(torch, ar, nbytes: int, steps: int, warmup: int):
    """Plain device copy of `nbytes` (a one-rank all-gather: 16-byte loads
    and stores, src read once, dst written once). Returns (ms per copy,
    HBM GB/s counting read + write)."""
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    with ar.Comm(1, 0) as comm:
        def step():
            ar.ar_all_gather(comm, [src.data_ptr()], [dst.data_ptr()], nbytes // 4, "i32", "fused", stream)

        for _ in range(warmup):
            step()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(steps):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    assert torch.equal(src, dst)
    del src, dst
    torch.cuda.empty_cache()
    return ms, 2 * nbytes / (ms * 1e-3) / 1e9


def copy_probe(args, torch, ar):
    """Plain copy of a known size: src read once, dst written once."""
    nbytes = args.copy_probe
    ms, gbps = time_copy(torch, ar, nbytes, args.steps, args.warmup)
    print(json.dumps({"probe": "copy", "bytes": nbytes, "ms_per_copy": round(ms, 4), "hbm_gbps": round(gbps, 1),
                      "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "steps": args.steps}), flush=True)


SWEEP_MODES = ("fused", "stepwise", "graph", "tree", "tree_stepwise")
SWEEP_MAX_SETS = 64
SWEEP_MARKER = "spin_kernel"  # torch.cuda._sleep's kernel: separates the sweep's groups in a kernel trace


def sweep_launches(mode: str, n: int) -> int:
    """Kernel launches one in-place all-reduce call makes in each mode."""
    levels = (n - 1).bit_length()
    return {"fused": 1, "tree": 1, "tree_stepwise": 2 * levels}.get(mode, 2 * (n - 1))


def sweep(args, torch, ar, synthetic):
    """The alpha vs beta regimes: 8 ranks, 1 KiB .. 256 MiB per rank in powers
    of two, fp32 SUM, in place, each mode. One JSON line per (mode, size),
    then one line with the alpha-beta fits (alpha_beta_fit: alpha from the
    latency regime, beta from the HBM-bound sizes)
      ring modes: T = 2(N-1)*alpha + moved/beta, moved = 5(N-1)*S (the bytes
                  the N-1 reduce-scatter and N-1 all-gather steps move)
      fused:      T = alpha + 2*N*S/beta.
    The time per call is host events over back-to-back calls, so it includes
    what the host spends enqueueing a call when that exceeds the device time.
    Each (mode, size) group starts with a torch.cuda._sleep marker kernel, so
    a rocprofv3 kernel trace of the run gives each group's device time
    (--sweep-trace). --cold rotates buffer sets of at least 1 GiB (at most
    SWEEP_MAX_SETS sets) so that every call reads HBM; --sweep-iters caps the
    calls per group."""
    n = 8
    rows = []
    group = 0
    with ar.Comm(n, 0) as comm:
        for log2 in range(10, 29):
            s_bytes = 1 << log2
            count = s_bytes // 4
            # at most SWEEP_MAX_SETS sets: below 2 MiB per rank the rotation
            # covers less than 1 GiB and the calls are partly cache-resident
            sets = min(SWEEP_MAX_SETS, -(-ROTATE_BYTES // (n * s_bytes))) if args.cold else 1
            bufsets = [synthetic.rank_inputs("sweep", n, count, "f32", device="cuda", salt=log2 + 100 * k)
                       for k in range(sets)]
            ptrsets = [[b.data_ptr() for b in bufs] for bufs in bufsets]
            stream = torch.cuda.current_stream()
            for mode in SWEEP_MODES:
                cur = [0]

                def call():
                    p = ptrsets[cur[0] % sets]
                    cur[0] += 1
                    ar.ar_all_reduce(comm, p, p, count, "f32", "sum", mode, stream)
                torch.cuda.synchronize()
                torch.cuda._sleep(1)  # group marker for kernel traces
                for _ in range(5):
                    call()
                iters = max(20, min(2000, int(2e9 / (2 * n * s_bytes))))
                if args.sweep_iters:
                    iters = min(iters, args.sweep_iters)
                start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                start.record(stream)
                for _ in range(iters):
                    call()
                stop.record(stream)
                torch.cuda.synchronize()
                ms = start.elapsed_time(stop) / iters
                calls = 5 + iters
                # fused kinds read N*S and write N*S; the stepwise ring and
                # tree both move 5(N-1)*S (3(N-1)S reducing, 2(N-1)S copying)
                moved = 2 * n * s_bytes if mode in ("fused", "tree") else 5 * (n - 1) * s_bytes
                row = {"sweep": mode, "group": group, "bytes_per_rank": s_bytes, "us": round(ms * 1e3, 3),
                       "iters": iters, "calls": calls, "launches_per_call": sweep_launches(mode, n),
                       "rotating_buffer_sets": sets,
                       "algbw_gbps": round(s_bytes / (ms * 1e-3) / 1e9, 3),
                       "busbw_gbps": round(s_bytes / (ms * 1e-3) / 1e9 * 2 * (n - 1) / n, 3),
                       "moved_bytes": moved, "moved_gbps": round(moved / (ms * 1e-3) / 1e9, 1)}
                if mode in ("stepwise", "tree_stepwise"):
                    ar.ar_comm_set_step_timing(comm, True)
                    call()
                    steps = ar.ar_last_step_times_ms(comm)
                    ar.ar_comm_set_step_timing(comm, False)
                    row["step_us"] = [round(t * 1e3, 2) for t in steps]
                    row["calls"] = calls + 1
                rows.append(row)
                group += 1
                print(json.dumps(row), flush=True)
            del bufsets, ptrsets
            torch.cuda.empty_cache()
        torch.cuda.synchronize()
        torch.cuda._sleep(1)  # closes the last group
        torch.cuda.synchronize()
    fits = {}
    for mode in SWEEP_MODES:
        rs = [r for r in rows if r["sweep"] == mode]
        launches = sweep_launches(mode, n)
        alpha, beta = alpha_beta_fit([(r["bytes_per_rank"], r["moved_bytes"], r["us"] * 1e-6) for r in rs],
                                     launches, n)
        fits[mode] = {"alpha_us": round(alpha * 1e6, 3), "beta_gbps": round(beta / 1e9, 1) if beta else None,
                      "model": "T = %d*alpha + moved/beta" % launches,
                      "alpha_from": "sizes up to %d bytes per rank" % SWEEP_LATENCY_MAX,
                      "beta_from": "sizes with N*S above the %d MiB last-level cache" % (LLC_BYTES >> 20)}
    small = {m: min(r["us"] for r in rows if r["sweep"] == m) for m in SWEEP_MODES}
    print(json.dumps({"sweep_fit": fits, "smallest_call_us": small, "nranks": n, "dtype": "f32", "op": "sum",
                      "cold": bool(args.cold)}), flush=True)


def read_kernel_trace(path: str):
    """(name, start ns, end ns) of every dispatch in a rocprofv3 kernel_trace.csv,
    in start order."""
    import csv
    out = []
    with open(path, newline="", encoding="utf-8") as f:
        for rec in csv.DictReader(f):
            out.append((rec["Kernel_Name"], int(rec["Start_Timestamp"]), int(rec["End_Timestamp"])))
    out.sort(key=lambda x: x[1])
    return out


def sweep_trace_summary(trace, rows, nranks: int = 8):
    """Each sweep group's device time from a kernel trace of the sweep: the
    library's kernels (names in namespace ar::) between the group's marker and
    the next one (rocprofv3 prints them as "void ar::..."). Returns one dict per row with the kernel count found, the
    expected count (calls x launches per call) and, when they agree, the
    device time per call and per launch; plus the alpha-beta fits on device
    time."""
    groups, cur = [], None
    for name, t0, t1 in trace:
        if SWEEP_MARKER in name:
            cur = []
            groups.append(cur)
        elif cur is not None and (name.startswith("ar::") or name.startswith("void ar::")):
            cur.append(t1 - t0)
    out = []
    for r in rows:
        g = groups[r["group"]] if r["group"] < len(groups) else []
        want = r["calls"] * r["launches_per_call"]
        d = {"sweep": r["sweep"], "bytes_per_rank": r["bytes_per_rank"], "host_us": r["us"], "kernels": len(g),
             "expected_kernels": want}
        if len(g) == want and want:
            d["device_us"] = sum(g) / r["calls"] / 1e3
            d["device_us_per_launch"] = sum(g) / want / 1e3
        out.append(d)
    fits = {}
    for mode in SWEEP_MODES:
        pts = [(d["bytes_per_rank"], r["moved_bytes"], d["device_us"] * 1e-6)
               for d, r in zip(out, rows) if d["sweep"] == mode and "device_us" in d]
        if len(pts) == sum(1 for r in rows if r["sweep"] == mode) and pts:
            alpha, beta = alpha_beta_fit(pts, sweep_launches(mode, nranks), nranks)
            fits[mode] = {"alpha_device_us": alpha * 1e6, "beta_device_gbps": beta / 1e9 if beta else None}
    return out, fits


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="grad7b", choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default=None, choices=["fused", "stepwise", "graph", "tree", "tree_stepwise"],
                    help="default: stepwise for --workload small (the ring whose per-step cost it measures), "
                         "fused otherwise")
    ap.add_argument("--no-range", action="store_true",
                    help="skip the metric-range block (8 x 64 MiB, 8 x 256 MiB, the cold 25 MiB bucket) that "
                         "follows the default headline line")
    ap.add_argument("--collective", default="all_reduce",
                    choices=["all_reduce", "reduce_scatter", "all_gather", "all_to_all"],
                    help="the collective to time on the workload's rank buffers: reduce_scatter takes count "
                         "elements per rank in and count/N out, all_gather count/N in and count out, all_to_all "
                         "count in and out (out of place)")
    ap.add_argument("--op", default=None, choices=["sum", "avg", "max", "min", "prod"],
                    help="reduction op instead of the workload's own (all-reduce, reduce-scatter)")
    ap.add_argument("--multi", action="store_true",
                    help="bucket64/bucket8: reduce the bucket as its mixed-size tensors with ar_all_reduce_multi")
    ap.add_argument("--access", default="auto", choices=["auto", "streaming", "cached"],
                    help="access flavour of the one-launch calls (ar_comm_set_access): auto streams the all-reduce "
                         "above half the 256 MB last-level cache and the other collectives above all of it; "
                         "streaming always; cached whenever the footprint fits the cache")
    ap.add_argument("--streaming", action="store_true", help="the same as --access streaming")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line, sweep 1 KiB .. 256 MiB per rank (8 ranks, fp32 SUM) in every "
                         "mode and fit the alpha-beta model")
    ap.add_argument("--cold", action="store_true",
                    help="with --sweep: rotate buffer sets of at least 1 GiB so every call reads HBM")
    ap.add_argument("--sweep-iters", type=int, default=0, metavar="K",
                    help="with --sweep: at most K timed calls per (mode, size) (for profiled runs)")
    ap.add_argument("--sweep-trace", nargs=2, metavar=("KERNEL_TRACE_CSV", "SWEEP_JSONL"),
                    help="instead of running anything, attribute a rocprofv3 kernel trace of a --sweep run to its "
                         "(mode, size) groups and print each group's device time beside the host-event time, "
                         "with alpha-beta fits on both")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="instead of the all-reduce, time a plain 16-byte-vector device copy of BYTES bytes "
                         "(a one-rank all-gather): the practical HBM ceiling, and the reference reading for "
                         "the HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the N virtual ranks of this all-reduce live on one "
              f"GPU as separate HBM buffers, and no figure across several GPUs is produced. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.sweep_trace:
        trace = read_kernel_trace(args.sweep_trace[0])
        lines = [json.loads(ln) for ln in open(args.sweep_trace[1], encoding="utf-8") if ln.startswith("{")]
        rows = [r for r in lines if "sweep" in r]
        host_fit = next((r for r in lines if "sweep_fit" in r), None)
        out, fits = sweep_trace_summary(trace, rows)
        for d in out:
            print(json.dumps(d), flush=True)
        print(json.dumps({"device_fit": fits, "host_fit": host_fit["sweep_fit"] if host_fit else None}), flush=True)
        return

    import torch
    import ring_all_reduce_ar_amd as ar
    import synthetic

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args, torch, ar)
        return
    if args.sweep:
        sweep(args, torch, ar, synthetic)
        return
    if args.mode is None:
        args.mode = "stepwise" if args.workload == "small" else "fused"
    n, count, dtype, op, desc = WORKLOADS[args.workload]
    if args.op and args.op != op:
        op = args.op
        desc += f"; op {op.upper()} instead"
    wl = {"bucket8": "bucket64"}.get(args.workload, args.workload)
    wl = wl if wl in synthetic.WORKLOAD_IDS else "sweep"
    comm = ar.Comm(n, 0)
    if args.streaming:
        args.access = "streaming"
    ar.ar_comm_set_access(comm, args.access)
    stream = torch.cuda.current_stream()
    sizes = None
    coll = args.collective
    if coll != "all_reduce":
        if args.multi or args.mode not in ("fused", "stepwise", "graph") or count % n:
            print("bench.py: --collective other than all_reduce takes a ring mode, no --multi, and a count "
                  "divisible by the rank count", file=sys.stderr)
            sys.exit(2)
        desc += f"; {coll}, out of place"
    if args.multi:
        if args.workload not in ("bucket64", "bucket8") or args.mode != "fused":
            print("bench.py: --multi applies to --workload bucket64 or bucket8 in fused mode", file=sys.stderr)
            sys.exit(2)
        sizes = synthetic.bucket_sizes(count, ESIZE[dtype], 4096, 64 << 20, seed=5)
        desc += f"; as {len(sizes)} tensors per rank through ar_all_reduce_multi"
    if args.access != "auto":
        desc += f"; {args.access} access (ar_comm_set_access)"

    s_bytes = count * ESIZE[dtype]
    # A call whose rank buffers fit in the last-level cache would be timed
    # warm if it ran on one buffer set back to back; rotate K sets so that
    # K*N*S >= 1 GiB and every call reads from HBM. The warm figure on one
    # set is reported beside it, labelled.
    foot = {"all_reduce": n, "all_to_all": 2 * n}.get(coll, n + 1) * s_bytes  # distinct bytes per call
    sets = 1 if foot > LLC_BYTES else -(-ROTATE_BYTES // foot)

    def timed_pass(measure_warm: bool):
        """Allocate and fill the rank buffers, warm up, time exactly K steps
        between two events; then K more steps with an event after each for
        the per-step times."""
        print(f"[bench] generating {desc}" + (f" ({sets} rotating buffer sets)" if sets > 1 else ""),
              file=sys.stderr, flush=True)
        # the input side: count elements per rank, or count/N for all-gather
        in_count = count // n if coll == "all_gather" else count
        out_count = {"all_reduce": count, "reduce_scatter": count // n}.get(coll, count)
        bufsets = [synthetic.rank_inputs(wl, n, in_count, dtype, device="cuda", op=op, salt=k) for k in range(sets)]
        outsets = None if coll == "all_reduce" else \
            [[torch.empty(out_count, dtype=bufsets[0][0].dtype, device="cuda") for _ in range(n)] for _ in range(sets)]
        ws = None
        cenum = {"all_reduce": ar.AR_COLL_ALL_REDUCE, "reduce_scatter": ar.AR_COLL_REDUCE_SCATTER,
                 "all_gather": ar.AR_COLL_ALL_GATHER, "all_to_all": ar.AR_COLL_ALL_TO_ALL}[coll]
        wcount = count // n if coll == "reduce_scatter" else count
        need = ar.ar_workspace_bytes(cenum, n, wcount, dtype, args.mode)
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            ar.ar_comm_set_workspace(comm, ws)
        ptrsets = [[b.data_ptr() for b in bufs] for bufs in bufsets]
        outptrs = None if outsets is None else [[b.data_ptr() for b in bufs] for bufs in outsets]
        if coll != "all_reduce":
            def step(i):
                p, q = ptrsets[i % sets], outptrs[i % sets]
                if coll == "reduce_scatter":
                    ar.ar_reduce_scatter(comm, p, q, count // n, dtype, op, args.mode, stream)
                elif coll == "all_gather":
                    ar.ar_all_gather(comm, p, q, count // n, dtype, args.mode, stream)
                else:
                    ar.ar_all_to_all(comm, p, q, count // n, dtype, args.mode, stream)
        elif sizes is None:
            def step(i):
                p = ptrsets[i % sets]
                ar.ar_all_reduce(comm, p, p, count, dtype, op, args.mode, stream)
        else:
            offs = [0]
            for c in sizes[:-1]:
                offs.append(offs[-1] + c)
            rowsets = [[[p + o * ESIZE[dtype] for p in ptrs] for o in offs] for ptrs in ptrsets]

            def step(i):
                rows = rowsets[i % sets]
                ar.ar_all_reduce_multi(comm, rows, rows, sizes, dtype, op, "fused", stream)

        def run(k, rotate, per_step_events=False):
            return time_steps(torch, stream, step, k, args.warmup, rotate, per_step_events)

        print(f"[bench] timing {args.warmup} warmup + {args.steps} steps", file=sys.stderr, flush=True)
        ms_ = run(args.steps, True)[0]
        per_step = run(args.steps, True, per_step_events=True)[1]
        warm = run(args.steps, False)[0] if measure_warm and sets > 1 else None
        ring_steps = None
        if measure_warm and args.mode in ("stepwise", "tree_stepwise"):
            # events between the ring's launches (ar_comm_set_step_timing):
            # each launch's device time, over K calls
            ar.ar_comm_set_step_timing(comm, True)
            calls = []
            for i in range(args.steps):
                step(i)
                calls.append(ar.ar_last_step_times_ms(comm))
            ar.ar_comm_set_step_timing(comm, False)
            ring_steps = calls
        sbc = None
        if measure_warm and coll == "all_reduce" and sizes is None and s_bytes % 16 == 0:
            # the same bytes as a plain copy on these rank buffers (overwrites them)
            sbc = same_buffer_copy_ms(torch, ar, ptrsets[0], s_bytes, stream, steps=3)
        ar.ar_comm_set_workspace(comm, None)
        del bufsets, ptrsets, outsets, outptrs, ws
        torch.cuda.empty_cache()
        return ms_, per_step, warm, ring_steps, sbc

    # In the first process on a freshly started MI355X, the first allocation
    # of the rank buffers measured 3-7% slower than the same buffers allocated
    # again after a free to the driver (same virtual addresses): the same
    # requests, evenly spread over the L2 channels, with fewer of them in
    # flight toward memory. Both passes are timed; the second is the steady
    # state a long-running job sees and is the reported value; the first is
    # reported beside it.
    first_ms = timed_pass(False)[0]
    ms, per_step, warm_ms, ring_steps, sbc_ms = timed_pass(True)
    per_step.sort()

    # nccl-tests conventions: algbw = S / T with S the per-rank buffer of
    # count elements (the input of reduce-scatter and all-to-all, the output
    # of all-gather); busbw = algbw * 2(N-1)/N for all-reduce, (N-1)/N else.
    algbw = s_bytes / (ms * 1e-3) / 1e9
    busbw = algbw * (2 if coll == "all_reduce" else 1) * (n - 1) / n
    # Algorithmic HBM bytes per call: all-reduce and all-to-all read N*S and
    # write N*S; reduce-scatter reads N*S and writes S (N blocks of S/N);
    # all-gather reads S (N blocks of S/N) and writes N*S. Stepwise modes
    # move more and are reported against the same bytes, so modes compare.
    alg_bytes = (2 * n if coll in ("all_reduce", "all_to_all") else n + 1) * s_bytes
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    # counter summaries cover the default access rule and the flat call
    # the committed counters belong to the workload's own op, access and layout
    own = not args.multi and args.access == "auto" and op == WORKLOADS[args.workload][3]
    traffic = load_traffic(args.workload, args.mode, coll) if own else None
    result = {
        "metric": METRIC,
        "value": sig(algbw),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sig(ms),
        "first_allocation_ms_per_step": sig(first_ms),
        "step_ms": {"median": sig(per_step[len(per_step) // 2]), "min": sig(per_step[0]),
                    "max": sig(per_step[-1])},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": desc, "nranks": n, "count_per_rank": count, "bytes_per_rank": s_bytes, "op": op,
                   "mode": args.mode, "collective": coll,
                   "accumulate": "f32" if dtype in ("f16", "bf16") else dtype,
                   "access": args.access if args.access != "auto" else
                   "auto: non-temporal above half the last-level cache (all-reduce) or all of it (others)",
                   "parallelism": f"{n} virtual ranks on 1 GPU"},
        "busbw": sig(busbw),
        "hbm_gbps": sig(achieved),
        "hbm_frac": sig(achieved / HBM_PEAK_GBPS),
        "roofline": {"bound": "hbm", "achieved": sig(achieved), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": sig(achieved / HBM_PEAK_GBPS),
                     "traffic": traffic},
    }
    if coll == "all_reduce" and args.mode in ("stepwise", "graph"):
        moved = ring_moved_bytes(n, count, dtype)
        result["moved"] = {"bytes": moved, "gbps": sig(moved / (ms * 1e-3) / 1e9),
                           "frac": sig(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS),
                           "note": "bytes the 2(N-1) ring steps read and write, over the call's time"}
    if sets > 1:
        result["config"]["rotating_buffer_sets"] = sets
        result["cache_resident"] = {"ms_per_step": sig(warm_ms),
                                    "effective_gbps": sig(alg_bytes / (warm_ms * 1e-3) / 1e9),
                                    "note": "one buffer set called back to back; served from the last-level cache"}
    # A plain 1 GiB device copy in the same process: the practical ceiling of
    # a read-once write-once stream on this machine, reported beside the roofline.
    cms, cgbps = time_copy(torch, ar, COPY_CEILING_BYTES, 20, 3)
    result["copy_ceiling"] = {"bytes": COPY_CEILING_BYTES, "ms": sig(cms), "hbm_gbps": sig(cgbps),
                              "hbm_frac": sig(cgbps / HBM_PEAK_GBPS),
                              "achieved_over_copy": sig(achieved / cgbps)}
    if sbc_ms:
        # a copy that reads and writes each of the call's own rank buffers once
        # (rank r into rank r+1): the all-reduce's bytes on the same
        # allocations, whose placement in memory sets the rate of both
        result["same_buffer_copy"] = {"ms": sig(sbc_ms), "hbm_frac": sig(alg_bytes / (sbc_ms * 1e-3) / 1e9 /
                                                                          HBM_PEAK_GBPS),
                                      "achieved_over_copy": sig(sbc_ms / ms)}
    if ring_steps:
        # Per-launch device times of the ring (the alpha-beta model's steps:
        # geek-doc page "训练梯度同步与集合通信", section 四; handbook
        # "集合通信原语", section α-β 模型). At a few KiB per rank a step
        # moves almost nothing, so its time is the per-step alpha on the
        # device; the call time over its launches is what a caller pays per
        # step, host enqueue included.
        launches = len(ring_steps[0])
        med = [sorted(c[j] for c in ring_steps)[len(ring_steps) // 2] for j in range(launches)]
        result["ring_steps"] = {
            "launches": launches, "step_us_median": [sig(t * 1e3) for t in med],
            "alpha_device_us": sig(sum(med) / launches * 1e3),
            "alpha_call_us": sig(ms * 1e3 / launches),
            "note": "step_us: events between the launches of one call (median over K calls); alpha_device_us "
                    "their mean; alpha_call_us: ms_per_step over the launches (host enqueue included)"}
    if (args.workload == "grad7b" and coll == "all_reduce" and args.mode == "fused" and not args.multi
            and args.access == "auto" and not args.no_range):
        # the metric's range below the headline: 8 ranks x 64 MiB, 256 MiB and
        # the cold 25 MiB DDP bucket, against the same copy ceiling
        result["range"] = []
        for name, k in RANGE_POINTS:
            print(f"[bench] range point {name}", file=sys.stderr, flush=True)
            result["range"].append(range_point(torch, ar, synthetic, name, k, 10, cgbps))
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(n, dtype, op, args.workload, coll, count)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

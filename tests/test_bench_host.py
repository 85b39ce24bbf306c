"""Host-side logic of bench.py's CPU baseline: which sample of the workload the
oracle is timed on, and how a short sample is repeated."""
import bench


def test_cpu_baseline_takes_the_whole_workload_when_it_fits(monkeypatch):
    monkeypatch.setattr(bench, "CPU_MIN_SECONDS", 0.0)
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    r = bench.cpu_baseline(4, "f32", "sum", "sweep", "all_reduce", count=4096)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert "4 ranks x 4096 f32 elements per rank" in r["sample"]
    assert "the whole workload" in r["sample"]
    assert r["value"] > 0 and r["seconds"] > 0
    # the all-reduce runs on the host's threads, and the fold is timed beside it
    assert r["cores"] == 3 and "on 3 threads" in r["sample"]
    assert r["fold"]["cores"] == 3 and r["fold"]["value"] > 0


def test_cpu_threads_follow_the_host_share(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "16")
    assert bench.cpu_threads() == 16
    monkeypatch.delenv("OMP_NUM_THREADS")
    import os
    assert bench.cpu_threads() == len(os.sched_getaffinity(0))


def test_cpu_baseline_windows_a_larger_workload(monkeypatch):
    monkeypatch.setattr(bench, "CPU_MIN_SECONDS", 0.0)
    monkeypatch.setattr(bench, "CPU_WINDOW_LOG2", 10)
    r = bench.cpu_baseline(8, "f16", "avg", "grad7b", "reduce_scatter", count=7_000_000_000)
    assert "8 ranks x 1024 f16 elements per rank" in r["sample"]
    assert "a window of the 7000000000-element workload" in r["sample"]
    assert "reduce-scatter" in r["sample"]
    assert r["cores"] == 1 and "fold" not in r


def test_cpu_baseline_repeats_a_short_sample(monkeypatch):
    monkeypatch.setattr(bench, "CPU_MIN_SECONDS", 0.05)
    r = bench.cpu_baseline(2, "i32", "sum", "sweep", "all_gather", count=64)
    assert r["seconds"] >= 0.05
    assert r["sample"].endswith(" calls")
    calls = int(r["sample"].rsplit(", ", 1)[1].split()[0])
    # the rate counts every call: bytes per call x calls / time
    assert abs(r["value"] - 64 * 4 * calls / r["seconds"] / 1e9) <= 1e-9 * r["value"] + 1e-12


def _moved_by_steps(n, count, dtype):
    # walk the ring's steps and add up what each one reads and writes per element
    e = bench.ESIZE[dtype]
    half = dtype in ("f16", "bf16")
    total = 0
    for s in range(n - 1):  # reduce-scatter
        first, last = s == 0, s == n - 2
        if not half:
            total += 3 * e * count  # local + incoming read, partial written
        else:
            incoming = 2 if first else 4  # a neighbour's fp16 input, else its fp32 partial
            written = 2 if last else 4  # the fp16 result, else an fp32 partial
            total += (2 + incoming + written) * count
    total += (n - 1) * 2 * e * count  # all-gather copies
    return total


def test_ring_moved_bytes_matches_the_step_walk():
    for n in range(2, 10):
        for dtype in ("f32", "i32", "f16", "bf16"):
            for count in (1, 7, 4096, 1000003):
                assert bench.ring_moved_bytes(n, count, dtype) == _moved_by_steps(n, count, dtype), (n, dtype, count)
    # the figures quoted for 8 ranks: 35*S for fp32, 94*count with the fp32 workspace
    assert bench.ring_moved_bytes(8, 100, "f32") == 35 * 400
    assert bench.ring_moved_bytes(8, 100, "f16") == 94 * 100
    assert bench.ring_moved_bytes(1, 100, "f32") == 0


def test_traffic_follows_collective_and_source_hash(monkeypatch, tmp_path):
    """roofline.traffic comes from the counter summary of the same workload,
    mode and collective, and only while the kernel sources still have the
    hash recorded in it."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_w_fused.md").write_text("kernel_sha: abc123\ntraffic_bytes_per_launch: 2.5e+10\n")
    (prof / "traffic_w_fused_all_gather.md").write_text("kernel_sha: abc123\ntraffic_bytes_per_launch: 1.5e+10\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sha", lambda: "abc123")
    assert bench.load_traffic("w", "fused") == 2.5e10
    assert bench.load_traffic("w", "fused", "all_gather") == 1.5e10
    assert bench.load_traffic("w", "fused", "reduce_scatter") is None
    assert bench.load_traffic("w", "stepwise") is None
    monkeypatch.setattr(bench, "kernel_sha", lambda: "def456")
    assert bench.load_traffic("w", "fused") is None


def test_sweep_trace_attribution(tmp_path):
    """Each sweep group's library kernels are the ones between its marker
    and the next; other kernels (torch's) are ignored; a group whose kernel
    count differs from calls x launches gets no device time."""
    rows = [
        {"sweep": "fused", "group": 0, "bytes_per_rank": 1024, "us": 5.0, "calls": 3, "launches_per_call": 1,
         "moved_bytes": 16 * 1024},
        {"sweep": "stepwise", "group": 1, "bytes_per_rank": 1024, "us": 40.0, "calls": 2, "launches_per_call": 14,
         "moved_bytes": 35 * 1024},
        {"sweep": "tree", "group": 2, "bytes_per_rank": 1024, "us": 6.0, "calls": 2, "launches_per_call": 1,
         "moved_bytes": 16 * 1024},
    ]
    t = 0
    lines = ["Kernel_Name,Start_Timestamp,End_Timestamp"]

    def k(name, dur):
        nonlocal t
        lines.append(f'"{name}",{t},{t + dur}')
        t += dur + 10

    k("at::native::uniform_kernel", 500)
    k("at::cuda::(anonymous namespace)::spin_kernel(long)", 50)
    for _ in range(3):
        k("void ar::detail::fused_reduce_vec<...>(ar::ReduceArgs)", 2000)
    k("spin_kernel(long)", 50)
    k("at::native::fill_kernel", 70)
    for _ in range(2 * 14):
        k("ar::detail::rs_step<...>", 1000)
    k("spin_kernel(long)", 50)
    k("ar::detail::tree_fused_vec<...>", 3000)  # one of two calls missing
    k("spin_kernel(long)", 50)
    path = tmp_path / "kernel_trace.csv"
    path.write_text("\n".join(lines) + "\n")
    out, _ = bench.sweep_trace_summary(bench.read_kernel_trace(str(path)), rows)
    assert out[0]["kernels"] == 3 and abs(out[0]["device_us"] - 2.0) < 1e-9
    assert out[1]["kernels"] == 28 and abs(out[1]["device_us"] - 14.0) < 1e-9
    assert abs(out[1]["device_us_per_launch"] - 1.0) < 1e-9
    assert out[2]["kernels"] == 1 and "device_us" not in out[2]

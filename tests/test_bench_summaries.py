"""CPU tests of bench.py's measurement plumbing: the rocprofv3 summaries it writes into profiles/.

The counter summary keeps only the per-launch replays (the dispatches after the network's last
average-pool dispatch), scales each counter by what it reads for a copy of known size, and
averages per kernel instance; the trace summary does the same selection for launch durations.
Synthetic CSV files stand in for rocprofv3's output (same columns)."""
import csv
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

K1 = "void ifx::(anonymous namespace)::igemm_kernel<3, 3, 128, 128, 2, false, true, false>(ifx::ConvArgs, int)"
K2 = "void ifx::(anonymous namespace)::conv1x1_kernel<128, 128, 2, true, true>(ifx::ConvArgs, int)"
POOL = "avgpool_kernel(signed char const*, signed char*, long long, int)"
COPY = "void at::native::vectorized_elementwise_kernel<4, bitwise_not_kernel_cuda(at::TensorIteratorBase&)>"


def _write(path, fields, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_summary_keeps_replays_and_scales(tmp_path):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    kib = 1 << 10
    # forward dispatches (ids 1..3, before the pool at id 4) read other sizes and must be ignored
    fetch = [(1, K1, 999), (2, K2, 999), (3, K1, 999), (4, POOL, 5),
             (5, K1, 100), (6, K2, 300), (7, K1, 140),
             (8, COPY, 7), (9, COPY, 512), (10, COPY, 512), (11, COPY, 512)]
    write = [(i, k, v // 2) for i, k, v in fetch]
    _write(tmp_path / "f.csv", fields, [dict(zip(fields, (i, k, "FETCH_SIZE", v))) for i, k, v in fetch])
    _write(tmp_path / "w.csv", fields, [dict(zip(fields, (i, k, "WRITE_SIZE", v))) for i, k, v in write])
    out = tmp_path / "traffic.txt"
    calib = 1024 * kib                                   # the copy moves 1 MiB: fetch reads 512 KiB -> x2
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), calib, str(out), "net", "note")
    lines = {ln.split(" | ")[0]: ln for ln in out.read_text().splitlines() if ln.startswith("kernel: ")}
    k1 = lines["kernel: igemm_kernel<3, 3, 128, 128, 2, false, true, false>"]
    assert "dispatches=2 " in k1
    assert f"fetch_bytes_per_launch={120 * kib * 2} " in k1     # mean(100, 140) KiB x 2
    assert f"write_bytes_per_launch={60 * kib * 4}" in k1       # mean(50, 70) KiB x (1 MiB / 256 KiB)
    k2 = lines["kernel: conv1x1_kernel<128, 128, 2, true, true>"]
    assert f"hbm_bytes_per_launch={300 * kib * 2 + 150 * kib * 4}" in k2
    assert "calib_bytes=1048576 | fetch_read=524288 | write_read=262144" in out.read_text()


def test_trace_summary_replay_averages(tmp_path):
    tf = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    trace = [(1, K1, 0, 900), (2, POOL, 1000, 1100),
             (3, K1, 2000, 2100), (4, K2, 3000, 3300), (5, K1, 4000, 4300)]
    _write(tmp_path / "t.csv", tf, [dict(zip(tf, r)) for r in trace])
    sf = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"]
    _write(tmp_path / "s.csv", sf, [dict(zip(sf, (K1, 3, 1300, 433.3, 70.0, 100, 900)))])
    out = tmp_path / "stats.txt"
    bench.summarize_trace(str(tmp_path / "t.csv"), str(tmp_path / "s.csv"), str(out), "net", "note")
    text = out.read_text()
    assert "igemm_kernel<3, 3, 128, 128, 2, false, true, false>(ifx::ConvArgs, int) | 3 | 433 | 1300" in text
    assert "replay: igemm_kernel<3, 3, 128, 128, 2, false, true, false> | 2 | 200 | 100 | 300" in text
    assert "replay: conv1x1_kernel<128, 128, 2, true, true> | 1 | 300 | 300 | 300" in text


def test_kernel_names_match_the_profiled_instances():
    """The library's kernel-name query (the launch's own dispatch, run without launching) names
    exactly the kernel instances rocprofv3 recorded for the network's per-launch replays in
    profiles/kernel_stats_net.txt (the FC's instance may appear there too)."""
    import convolution_int8_implicit_amd as ifx
    from convolution_int8_implicit_amd import synth
    names = set(bench.net_kernel_names(synth.workload(4).net, 1024))
    fc = ifx.conv_kernel_name(ifx.conv_desc(1024, 1, 1, 2048, 1000, 1, 1, 1, 0, ifx.OUT_I32))
    with open(os.path.join(ROOT, "profiles", "kernel_stats_net.txt")) as fh:
        profiled = {ln.split(" | ")[0][len("replay: "):] for ln in fh if ln.startswith("replay: ")}
    assert names <= profiled, names - profiled
    assert profiled <= names | {fc}, profiled - names

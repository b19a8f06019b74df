"""The rocprofv3 summariser (paged_kv_cache_64_amd/prof_summary.py) on small
synthetic CSV files: kernel statistics, counter scaling against a plain copy,
and the counter file that bench.py reads traffic from."""
import os

import bench
from paged_kv_cache_64_amd import prof_summary as ps


def _write(path, header, rows):
    """A CSV file as rocprofv3 writes them (fields with commas quoted)."""
    import csv

    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def _counters(d, counter, per_kernel):
    _write(os.path.join(d, "run", "x_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
           [(k, counter, v) for k, vals in per_kernel.items() for v in vals])


def test_trace_orders_kernels_by_total_time(tmp_path):
    _write(str(tmp_path / "t" / "a_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
           [("small_kernel", 10, 100, 10, 1, 9, 11, 0), ("big_kernel", 4, 4000, 1000, 99, 900, 1100, 0)])
    rows = ps.kernel_stats(str(tmp_path / "t"))
    assert [r[0] for r in rows] == ["big_kernel", "small_kernel"]
    assert rows[0][1:] == (4, 1000.0, 900.0, 1100.0, 4000.0)


def test_counters_scale_by_the_copy_and_match_the_kernel_source(tmp_path, monkeypatch):
    cal_bytes = 1 << 20
    # the copy reads half its bytes in FETCH_SIZE and all of them in WRITE_SIZE (KiB)
    _counters(str(tmp_path / "cf"), "FETCH_SIZE", {"probe_copy_kernel(x)": [512.0, 512.0]})
    _counters(str(tmp_path / "cw"), "WRITE_SIZE", {"probe_copy_kernel(x)": [1024.0]})
    # two instantiations of the kernel: weighted by dispatches
    _counters(str(tmp_path / "f"), "FETCH_SIZE", {"k<1>(a)": [100.0, 100.0, 100.0], "k<2>(a)": [200.0],
                                                  "other(a)": [9.0]})
    _counters(str(tmp_path / "w"), "WRITE_SIZE", {"k<1>(a)": [10.0]})
    out = tmp_path / "c.txt"
    ps.main(["-o", str(out), "counters", "--kernel", "k<", "--fetch", str(tmp_path / "f"),
             "--write", str(tmp_path / "w"), "--cal-fetch", str(tmp_path / "cf"), "--cal-write",
             str(tmp_path / "cw"), "--cal-bytes", str(cal_bytes), "--bytes", "256000", "--title", "t",
             "--workload", "w", "--command-fetch", "cf", "--command-write", "cw", "--command-cal", "cc"])
    text = out.read_text()
    fetch = (3 * 100.0 + 200.0) / 4 * 1024 * 2.0   # mean KiB x 1024 x fetch scale 2
    write = 10.0 * 1024 * 1.0
    assert f"fetch_bytes_per_launch: {fetch:.0f}" in text
    assert f"write_bytes_per_launch: {write:.0f}" in text
    assert "fetch_scale: 2.000000" in text and "write_scale: 1.000000" in text
    assert f"kernel_code_sha256: {bench.kernel_code_hash()}" in text
    assert bench.read_counter_file(str(out)) == int(fetch) + int(write)
    # a summary taken on other kernel source is not used
    monkeypatch.setattr(bench, "kernel_code_hash", lambda: "0" * 64)
    assert bench.read_counter_file(str(out)) is None


def test_sq_lists_every_counter_of_the_kernel(tmp_path):
    d = str(tmp_path / "s")
    _write(os.path.join(d, "run", "s_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
           [("k(a)", "SQ_WAVES", 8), ("k(a)", "SQ_WAVES", 4), ("k(a)", "SQ_BUSY_CYCLES", 100)])
    lines = ps.main(["-o", str(tmp_path / "sq.txt"), "sq", d, "--kernel", "k("]) or \
        (tmp_path / "sq.txt").read_text().splitlines()
    assert "k( SQ_BUSY_CYCLES: 100 per launch over 1 launches" in lines
    assert "k( SQ_WAVES: 6 per launch over 2 launches" in lines
    assert f"# kernel_code_sha256: {bench.kernel_code_hash()}" in lines


def test_dispatch_trace_skips_warmup_and_reports_the_median(tmp_path):
    hdr = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows = []
    t = 0
    # decode: 3 slow warm-up dispatches, then 5 timed ones (100, 102, 98, 101, 99 ns)
    for i, dur in enumerate([500, 400, 300, 100, 102, 98, 101, 99]):
        rows.append(("KERNEL_DISPATCH", 10 + 2 * i, "decode_partial_kernel<3, false>", t, t + dur))
        t += 1000
    rows.append(("KERNEL_DISPATCH", 11, "write_kv_kernel", 5, 25))
    # out of order in the file: sorted by dispatch id
    _write(str(tmp_path / "tr" / "x_kernel_trace.csv"), hdr, rows[::-1])
    got = ps.dispatch_stats(str(tmp_path / "tr"), {"decode_partial": 3})
    by = {r[0]: r for r in got}
    d = by["decode_partial_kernel<3, false>"]
    assert d[1] == 5 and d[2] == 100.0 and d[3] == 100 and d[4] == 98 and d[5] == 102 and d[7] == 3
    assert by["write_kv_kernel"][1:4] == (1, 20.0, 20)
    ps.main(["-o", str(tmp_path / "out.txt"), "trace", str(tmp_path / "tr"), "--title", "T", "--command", "C",
             "--skip", "decode_partial=3"])
    out = open(tmp_path / "out.txt").read()
    assert "first 3 dispatches" in out and "median ns" in out
    assert f"# kernel_code_sha256: {bench.kernel_code_hash()}" in out.splitlines()
    assert ps.dispatch_stats(str(tmp_path / "none")) is None


def test_bench_names_the_kernels_a_decode_launch_runs():
    from types import SimpleNamespace as NS
    assert bench.launch_kernels(NS(num_items=32, num_prefix_items=0, num_merges=0, max_piece_tokens=4096,
                                   decode_wave_heads=0)) == "decode_partial_kernel"
    assert bench.launch_kernels(NS(num_items=40, num_prefix_items=0, num_merges=3, max_piece_tokens=1024,
                                   decode_wave_heads=0)) == \
        "decode_partial_kernel + decode_merge_planned_kernel"
    # many short pieces: each wave walks a piece for its own KV head
    assert bench.launch_kernels(NS(num_items=1024, num_prefix_items=0, num_merges=0, max_piece_tokens=128,
                                   decode_wave_heads=1)) == "decode_wave_heads_kernel"
    assert bench.launch_kernels(NS(num_items=1024, num_prefix_items=0, num_merges=0, max_piece_tokens=128,
                                   decode_wave_heads=1), num_kv_heads=2) == "decode_partial_kernel"
    # ordinary and shared-prefix pieces run in one cascade launch, then the merge
    assert bench.launch_kernels(NS(num_items=340, num_prefix_items=64, num_merges=256)) == \
        "cascade_kernel + decode_merge_planned_kernel"
    assert bench.launch_kernels(NS(num_items=0, num_prefix_items=8, num_merges=4, max_piece_tokens=0)) == \
        "decode_prefix_kernel + decode_merge_planned_kernel"

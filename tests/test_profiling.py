"""Host-side summaries of rocprofv3 output (head_latent_attention_04_amd.profiling), on small
hand-written CSV files in rocprofv3's column layout: the back-to-back dispatch run and the
copy-calibrated HBM traffic that bench.py reports."""
import csv

from head_latent_attention_04_amd import profiling

TRACE_COLS = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
COUNTER_COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, cols, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_backtoback_takes_the_longest_run_of_one_kernel(tmp_path):
    # dispatch order (ids deliberately shuffled in the file): A A B A A A B A; durations in ns
    seq = [("A", 40_000), ("A", 50_000), ("B", 9_000), ("A", 42_000), ("A", 44_000), ("A", 46_000), ("B", 9_000),
           ("A", 99_000)]
    rows, t = [], 1_000_000
    for i, (k, d) in enumerate(seq):
        rows.append(("KERNEL_DISPATCH", i + 1, f"void ns::{k}_kernel<4>(int)", t, t + d))
        t += d + 500
    rows.reverse()
    p = tmp_path / "run_kernel_trace.csv"
    _write(p, TRACE_COLS, rows)
    line = profiling.backtoback(str(p), "A_kernel")
    assert "longest back-to-back run 3 dispatches" in line
    assert "average 44.00 us" in line and "min 42.00" in line and "max 46.00" in line


def test_traffic_scales_each_counter_by_the_copy_reading(tmp_path):
    copy_bytes = 1 << 20
    # the counters read 2x the bytes for a copy of 1 MiB (read 1 MiB, write 1 MiB): 2048 KiB each
    fetch = [(1, "copyBuffer", "FETCH_SIZE", 2048.0), (2, "attn_kernel<1>", "FETCH_SIZE", 100.0),
             (3, "attn_kernel<1>", "FETCH_SIZE", 300.0), (4, "other", "FETCH_SIZE", 5.0)]
    write = [(1, "copyBuffer", "WRITE_SIZE", 4096.0), (2, "attn_kernel<1>", "WRITE_SIZE", 64.0)]
    fp, wp = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write(fp, COUNTER_COLS, fetch)
    _write(wp, COUNTER_COLS, write)
    res = profiling.traffic(str(fp), str(wp), "attn_kernel", "w", copy_bytes, "cmd")
    # fetch: average 200 KiB, factor 1 MiB / 2048 KiB = 0.5 -> 102400 B; write: 64 KiB x 0.25 -> 16384 B
    assert res["FETCH_SIZE"]["scale_factor"] == 0.5 and res["FETCH_SIZE"]["bytes_per_launch"] == 102400
    assert res["WRITE_SIZE"]["scale_factor"] == 0.25 and res["WRITE_SIZE"]["bytes_per_launch"] == 16384
    assert res["bytes_per_launch"] == 102400 + 16384
    assert res["workload"] == "w" and len(res["kernel_source_sha256_16"]) == 16

"""Host logic of the rocprofv3 summaries (no GPU): counter averaging per
dispatch, the sum over a sequence of kernels, and the copy-scaled HBM traffic
record that bench.py reports."""
import csv
import json

import pytest

from exact_attention_forward_02_amd import profiling

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, k, c, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_read_counters_sums_within_a_dispatch_and_averages_over_dispatches(tmp_path):
    p = tmp_path / "c.csv"
    # two dispatches of the kernel, each reported as two partial rows (e.g. per XCD)
    write_counters(p, [(1, "k_a<1>", "FETCH_SIZE", 10), (1, "k_a<1>", "FETCH_SIZE", 30),
                       (2, "k_a<1>", "FETCH_SIZE", 50), (2, "k_a<1>", "FETCH_SIZE", 70),
                       (3, "other", "FETCH_SIZE", 1000)])
    mean, n, name = profiling.read_counters(str(p), "k_a")
    assert n == 2 and name == "k_a<1>"
    assert mean["FETCH_SIZE"] == pytest.approx((40 + 120) / 2)


def test_read_counters_sum_adds_each_kernel_mean(tmp_path):
    p = tmp_path / "c.csv"
    write_counters(p, [(1, "x_delta", "WRITE_SIZE", 4), (2, "x_main", "WRITE_SIZE", 100),
                       (3, "x_delta", "WRITE_SIZE", 6), (4, "x_main", "WRITE_SIZE", 300),
                       (5, "x_tail", "WRITE_SIZE", 7), (6, "x_tail", "WRITE_SIZE", 9)])
    total, counts = profiling.read_counters_sum(str(p), "x_delta,x_main,x_tail")
    assert counts == [2, 2, 2]
    assert total["WRITE_SIZE"] == pytest.approx(5 + 200 + 8)
    with pytest.raises(SystemExit):
        profiling.read_counters_sum(str(p), "x_delta,missing")


def test_traffic_record_scales_by_the_copy_kernel(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    cfetch, cwrite = tmp_path / "cf.csv", tmp_path / "cw.csv"
    write_counters(fetch, [(1, "k_one", "FETCH_SIZE", 1000), (2, "k_two", "FETCH_SIZE", 500)])
    write_counters(write, [(1, "k_one", "WRITE_SIZE", 200), (2, "k_two", "WRITE_SIZE", 100)])
    # the copy kernel moved 1 MiB each way; FETCH_SIZE reads half of that
    write_counters(cfetch, [(1, "neg_kernel", "FETCH_SIZE", 512)])
    write_counters(cwrite, [(1, "neg_kernel", "WRITE_SIZE", 1024)])
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel source\n")
    out = tmp_path / "rec.json"
    profiling.main(["traffic", "--fetch", str(fetch), "--write", str(write),
                    "--copy-fetch", str(cfetch), "--copy-write", str(cwrite),
                    "--copy-bytes", str(1 << 20), "--kernel", "k_one,k_two",
                    "--source", str(src), "--workload", "w", "--out", str(out)])
    rec = json.loads(out.read_text())
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_read_bytes_per_launch"] == pytest.approx(1500 * 1024 * 2.0)
    assert rec["hbm_write_bytes_per_launch"] == pytest.approx(300 * 1024)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(1500 * 2048 + 300 * 1024)
    assert rec["kernel_source_sha256"] == profiling.kernel_source_digest(str(src))

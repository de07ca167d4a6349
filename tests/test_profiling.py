"""Host logic behind the bench's traffic figure and the trace summaries: the
rocprofv3 CSV readers, the copy calibration of FETCH_SIZE / WRITE_SIZE, and the
per-call sums. Synthetic CSVs in rocprofv3's column layout; no GPU."""
import csv
import json

import pytest

from top_selection_row_amd import profiling

PART = "void ds::deepselect_ring_kernel<ds::BF16P, 8, 4>(ds::Params)"
MERGE = "void ds::deepselect_merge_kernel<ds::BF16T, 8>(ds::Params)"
COPY = "__amd_rocclr_copyBuffer"


def write_counters(d, rows):
    d.mkdir(parents=True, exist_ok=True)
    with open(d / "pmc_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, name, counter, value in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})
    return d


def test_counters_sum_instances_then_average_dispatches(tmp_path):
    # two dispatches of the part kernel, each reported as two instances
    d = write_counters(tmp_path / "k", [(1, PART, "FETCH_SIZE", 10.0), (1, PART, "FETCH_SIZE", 30.0),
                                        (2, PART, "FETCH_SIZE", 50.0), (2, PART, "FETCH_SIZE", 10.0),
                                        (3, COPY, "FETCH_SIZE", 999.0)])
    got = profiling.counters(str(d))
    assert got == {"ds::deepselect_ring_kernel<ds::BF16P, 8, 4>": {"FETCH_SIZE": 50.0}}


def test_traffic_scales_by_the_copy_and_sums_the_kernels(tmp_path):
    copy_bytes = 512 * 2**20
    # the copy's FETCH_SIZE reads half of the bytes copied, WRITE_SIZE all of them
    cf = write_counters(tmp_path / "cf", [(1, COPY, "FETCH_SIZE", copy_bytes / 2 / 1024)])
    cw = write_counters(tmp_path / "cw", [(1, COPY, "WRITE_SIZE", copy_bytes / 1024)])
    kf = write_counters(tmp_path / "kf", [(1, PART, "FETCH_SIZE", 1000.0), (2, MERGE, "FETCH_SIZE", 100.0)])
    kw = write_counters(tmp_path / "kw", [(1, PART, "WRITE_SIZE", 40.0), (2, MERGE, "WRITE_SIZE", 8.0)])
    out = tmp_path / "t.json"
    profiling.main(["traffic", "--workload", "w", "--kernel-fetch", str(kf), "--kernel-write", str(kw),
                    "--copy-fetch", str(cf), "--copy-write", str(cw), "--copy-bytes", str(copy_bytes),
                    "--out", str(out)])
    d = json.load(open(out))
    assert d["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert d["copy_calibration"]["write_scale"] == pytest.approx(1.0)
    assert d["fetch_bytes_per_launch"] == pytest.approx((1000.0 + 100.0) * 1024 * 2)
    assert d["write_bytes_per_launch"] == pytest.approx((40.0 + 8.0) * 1024)
    assert d["hbm_bytes_per_launch"] == pytest.approx(d["fetch_bytes_per_launch"] + d["write_bytes_per_launch"])
    assert d["source_digest"] == profiling.source_digest()


def test_trace_per_call_total(tmp_path, capsys):
    d = tmp_path / "tr"
    d.mkdir()
    with open(d / "trace_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                                          "MaxNs"])
        w.writeheader()
        for name, calls, avg in [(PART, 10, 44000.0), (MERGE, 10, 9000.0), (COPY, 2, 11000.0)]:
            w.writerow({"Name": name, "Calls": calls, "TotalDurationNs": calls * avg, "AverageNs": avg,
                        "Percentage": 0.0, "MinNs": avg, "MaxNs": avg})
    profiling.main(["trace", str(d), "--title", "t"])
    text = capsys.readouterr().out
    assert "per call (deepselect_ring_kernel + deepselect_merge_kernel, 10 calls): 53.00 us" in text


def test_source_digest_is_stable():
    assert profiling.source_digest() == profiling.source_digest()
    assert len(profiling.source_digest()) == 16


def test_bench_w_bound_matches_the_model():
    # bench.py states the bound for its report; the oracle's model is the pinned one
    import bench
    from oracle import model

    for n, k, b, b2, split in [(4096, 64, 256, 256, 1), (131072, 2048, 2048, 2048, 2), (32768, 512, 1024, 1024, 4),
                               (1048576, 512, 1024, 1024, 16), (151936, 64, 1024, 1024, 1), (4097, 16, 256, 128, 3)]:
        assert bench.w_bound_row(n, k, b, b2, split) == pytest.approx(
            model.expected_w_bound_row(n, k, b, b2, split), rel=1e-12)


def test_sq_ratios():
    cs = {"SQ_WAVES": 4.0, "SQ_WAVE_CYCLES": 1000.0, "SQ_INSTS_VALU": 400.0, "SQ_ACTIVE_INST_VALU": 200.0,
          "SQ_THREAD_CYCLES_VALU": 6400.0, "SQ_ACTIVE_INST_LDS": 50.0, "SQ_LDS_BANK_CONFLICT": 25.0,
          "SQ_WAIT_ANY": 600.0}
    d = profiling.sq_derived(cs)
    assert d["insts_valu_per_wave"] == 100.0
    assert d["valu_active_share"] == 0.2
    assert d["valu_lane_utilisation"] == 0.5
    assert d["lds_bank_conflict_per_active_cycle"] == 0.5
    assert d["wait_any_share"] == 0.6

"""The rocprofv3 summaries behind profiles/: traffic scaling and the derived
counter figures, on small synthetic CSV files of rocprofv3's layout."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from chunked_attention_amd import profiling as P  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
          "End_Timestamp"]
ATTN_NAME = "void kvc::attn::attn_fwd_bf16<128, false, false, false>(kvc::attn::AttnArgs)"


def write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_traffic_scales_each_counter_by_the_copy_kernel(tmp_path):
    mib = 4
    # the copy kernel reads and writes 4 MiB: FETCH reads back 2 MiB (scale 2),
    # WRITE 4 MiB (scale 1); attention dispatches: only the last 2 count
    write_counters(tmp_path / "f", [
        (1, "neg_kernel", "FETCH_SIZE", 2048, 0, 1),
        (2, ATTN_NAME, "FETCH_SIZE", 999999, 0, 1),        # early, window filling
        (3, ATTN_NAME, "FETCH_SIZE", 600, 0, 1),
        (3, ATTN_NAME, "FETCH_SIZE", 400, 0, 1),           # a second instance: summed
        (4, ATTN_NAME, "FETCH_SIZE", 1000, 0, 1),
    ])
    write_counters(tmp_path / "w", [
        (1, "neg_kernel", "WRITE_SIZE", 4096, 0, 1),
        (3, ATTN_NAME, "WRITE_SIZE", 100, 0, 1),
        (4, ATTN_NAME, "WRITE_SIZE", 300, 0, 1),
    ])
    res, total = P.traffic(str(tmp_path / "f"), str(tmp_path / "w"), mib, steady=2)
    assert res["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert res["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    assert res["FETCH_SIZE"]["attn_bytes"] == pytest.approx(1000 * 1024 * 2)
    assert res["WRITE_SIZE"]["attn_bytes"] == pytest.approx(200 * 1024)
    assert total == pytest.approx(1000 * 1024 * 2 + 200 * 1024)


def test_counter_summary_derives_mfma_busy_and_its_algorithmic_share(tmp_path):
    # one dispatch of 100 us; GRBM_GUI_ACTIVE over 8 XCDs -> 200000 cycles
    # (2.00 GHz); matrix pipes busy for half of 1024 SIMDs x 200000 cycles
    cycles = 200_000
    busy = 0.5 * P.CUS * P.SIMDS * cycles
    flops = 0.25 * busy * P.BF16_FLOPS_PER_SIMD_CYCLE     # a quarter of the busy cycles
    write_counters(tmp_path / "a", [
        (7, ATTN_NAME, "GRBM_GUI_ACTIVE", cycles * P.XCDS, 0, 100_000),
        (7, ATTN_NAME, "SQ_VALU_MFMA_BUSY_CYCLES", busy / 2, 0, 100_000),
        (7, ATTN_NAME, "SQ_VALU_MFMA_BUSY_CYCLES", busy / 2, 0, 100_000),
        (8, "cache_write", "GRBM_GUI_ACTIVE", 1, 0, 5),
    ])
    write_counters(tmp_path / "b", [
        (7, ATTN_NAME, "SQ_INSTS_LDS", 1000, 0, 100_000),
        (7, ATTN_NAME, "SQ_LDS_BANK_CONFLICT", 250, 0, 100_000),
        (7, ATTN_NAME, "TCC_HIT_sum", 90, 0, 100_000),
        (7, ATTN_NAME, "TCC_MISS_sum", 10, 0, 100_000),
    ])
    md = P.counters_md([str(tmp_path / "a"), str(tmp_path / "b")], ["cmd a", "cmd b"],
                       steady=1, flops=flops, workload="test")
    assert "2.00 GHz" in md
    assert "= 50.0%." in md
    assert ": 25.0% of the busy cycles" in md
    assert "per LDS instruction: 0.250." in md
    assert "L2 hit rate: 90.0%." in md
    assert "Mean dispatch time in these runs: 100.0 us." in md
    assert "cmd a" in md and "cmd b" in md


def test_kernel_stats_summary_and_steady_mean(tmp_path):
    d = tmp_path / "s"
    os.makedirs(d)
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "MinNs", "MaxNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": ATTN_NAME, "Calls": 3, "TotalDurationNs": 600000,
                    "AverageNs": 200000, "MinNs": 100000, "MaxNs": 300000, "Percentage": 90.0})
        w.writerow({"Name": "void kvc::cache_write_bf16<128>(...)", "Calls": 6,
                    "TotalDurationNs": 66000, "AverageNs": 11000, "MinNs": 10000,
                    "MaxNs": 12000, "Percentage": 10.0})
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        # three attention calls (100, 300, 200 us) and a cache write between
        for start, dur in ((0, 100000), (400000, 300000), (900000, 200000)):
            w.writerow({"Kernel_Name": ATTN_NAME, "Start_Timestamp": start,
                        "End_Timestamp": start + dur})
        w.writerow({"Kernel_Name": "cache_write_bf16", "Start_Timestamp": 200000,
                    "End_Timestamp": 211000})
    md = P.stats_md(str(d), "the command", steady=2)
    assert "the command" in md
    assert "| attn_fwd_bf16<128, false, false, false> | 3 | 600.0 | 200.00 |" in md
    assert "| cache_write | 6 | 66.0 | 11.00 |" in md
    # the last two attention calls in time order: 300 and 200 us
    assert "mean 250.00 us per call" in md

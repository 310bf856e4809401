"""The rocprofv3 summariser (host logic, no GPU): kernel-name shortening, the stats
table, and the traffic record's scaling by the calibration kernel's readings."""
import csv
import json

import pytest

from paged_attention_decode_kv_amd import profiling as pf

DECODE = "void pkv::decode_kernel<unsigned short, 128, 8, true, 1>(pkv::AttnArgs, pkv::Workspace, float)"
CAL = ("void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, "
       "float, at::native::binary_internal::MulFunctor<float> >, std::array<char*, 2ul> >(int, ...)")


def test_short_name_keeps_template_arguments():
    assert pf.short_name(DECODE) == "pkv::decode_kernel<unsigned short, 128, 8, true, 1>"
    assert pf.short_name("pkv::plan_kernel(pkv::AttnArgs, pkv::Workspace)") == "pkv::plan_kernel"


def test_stats_rows_of_the_library_only(tmp_path):
    p = tmp_path / "stats.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        w.writerow([DECODE, 4, 4000000, 1000000, 90, 990000, 1010000, 1])
        w.writerow(["void at::native::something(int)", 2, 10, 5, 1, 4, 6, 1])
        w.writerow(["pkv::plan_kernel(pkv::AttnArgs, pkv::Workspace)", 4, 28000, 7000, 1, 6000,
                    8000, 1])
    rows = pf.kernel_stats(str(p))
    assert [r["kernel"] for r in rows] == ["pkv::decode_kernel<unsigned short, 128, 8, true, 1>",
                                           "pkv::plan_kernel"]
    assert rows[0]["avg_us"] == pytest.approx(1000.0)
    table = pf.stats_table(rows)
    assert "| `pkv::plan_kernel` | 4 | 7.00 | 6.00 | 8.00 |" in table


def _counters(path, counter, values):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for name, v in values:
            w.writerow([name, counter, v])


def test_traffic_scales_each_counter_by_the_calibration(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # the 1 GiB multiply: FETCH_SIZE counts half the bytes read, WRITE_SIZE all written
    _counters(fetch, "FETCH_SIZE", [(CAL, 524288.0)] * 3 + [(DECODE, 1000.0), (DECODE, 1002.0)])
    _counters(write, "WRITE_SIZE", [(CAL, 1048576.0)] * 3 + [(DECODE, 10.0), (DECODE, 10.0)])
    rec = pf.traffic_record(str(fetch), str(write), kernel="pkv::decode_kernel<",
                            workload="w", layout="HND", tag="t", algorithmic_bytes=2_000_000,
                            commands=["rocprofv3 --pmc FETCH_SIZE -- python3 bench.py"])
    assert rec["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["calibration"]["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes"] == round(1001.0 * 1024 * 2)
    assert rec["write_bytes"] == 10 * 1024
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["traffic_over_algorithmic"] == pytest.approx(rec["bytes_per_launch"] / 2e6)
    assert rec["kernel_source_sha256"] == pf.kernel_source_hash()
    # a second kernel matching the substring is refused rather than guessed
    _counters(fetch, "FETCH_SIZE", [(CAL, 524288.0), (DECODE, 1.0),
                                    (DECODE.replace("1>", "2>"), 1.0)])
    with pytest.raises(SystemExit):
        pf.traffic_record(str(fetch), str(write), kernel="pkv::decode_kernel<", workload="w",
                          layout="HND", tag="t", algorithmic_bytes=1, commands=[])


def test_update_replaces_the_record_of_the_same_workload_and_layout(tmp_path):
    path = tmp_path / "traffic.json"
    pf.update_records({"workload": "a", "layout": "HND", "x": 1}, str(path))
    pf.update_records({"workload": "a", "layout": "NHD", "x": 2}, str(path))
    pf.update_records({"workload": "a", "layout": "HND", "x": 3}, str(path))
    recs = json.loads(path.read_text())["records"]
    assert sorted((r["layout"], r["x"]) for r in recs) == [("HND", 3), ("NHD", 2)]

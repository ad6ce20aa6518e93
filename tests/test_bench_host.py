"""Host-side logic of bench.py (no GPU): the one-GPU contract, the counter
records' tie to the kernel sources, the rocprofv3 summaries, workload names."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_records_follow_the_kernel_sources(monkeypatch):
    recs = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    key = "ivfpq_n1m_d128_m16_nlist1024:f32"
    rec = recs[key]
    # a record applies while the sources hash to the digest it was taken on
    monkeypatch.setattr(bench, "source_digest", lambda: rec["source_sha256"])
    want = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert bench.stored_traffic(*key.split(":")) == want
    assert rec["fetch_bytes_per_launch"] == pytest.approx(
        rec["raw_kib_per_dispatch"]["FETCH_SIZE"] * 1024 * rec["calibration"]["read_factor"])
    # another kernel version retires them
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 64)
    assert bench.stored_traffic(*key.split(":")) is None
    assert bench.stored_traffic("no_such_workload", "f32") is None


def test_summaries_of_rocprof_csv(tmp_path, capsys):
    stats = tmp_path / "ks_kernel_stats.csv"
    stats.write_text('"Name","Calls","TotalDurationNs","AverageNs"\n'
                     '"void ivfpq::scan_items_kernel<8>(ivfpq::ScanArgs)",4,8000000,2000000\n')
    counters = tmp_path / "c_counter_collection.csv"
    counters.write_text('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n'
                        '1,"ivfpq::scan_items_kernel<8>(ivfpq::ScanArgs)","FETCH_SIZE",100\n'
                        '2,"ivfpq::scan_items_kernel<8>(ivfpq::ScanArgs)","FETCH_SIZE",300\n')
    bench.summarize_stats([str(stats)])
    bench.summarize_counters([str(counters)])
    out = capsys.readouterr().out
    assert "| `ivfpq::scan_items_kernel<8>` | 4 | 8.000 | 2000.0 |" in out
    assert "(2 dispatches, per dispatch): FETCH_SIZE=200" in out


def test_unknown_workload_is_named():
    with pytest.raises(SystemExit) as e:
        bench.workload("no_such_workload")
    assert "ivfpq_n1m_d128_m16_nlist1024" in str(e.value)

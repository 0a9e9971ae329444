"""bench.py on the host: the one-GPU contract and the traffic record lookup
(no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_traffic_is_used_only_for_the_current_kernel_source(tmp_path):
    h = bench.ffn_source_hash()
    assert len(h) == 16 and h == bench.ffn_source_hash()
    rec = {"mixtral_prefill": {"ffn_source": h, "fetch_bytes": 3.0e9, "write_bytes": 1.0e9}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(p), "mixtral_prefill") == 4.0e9
    assert bench.measured_traffic(str(p), "deepseek_v3") is None
    rec["mixtral_prefill"]["ffn_source"] = "0" * 16
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(p), "mixtral_prefill") is None
    assert bench.measured_traffic(str(tmp_path / "missing.json"), "mixtral_prefill") is None



def test_clock_summary_keeps_table_refreshes_seen_during_the_load():
    """The metrics table refreshes about once a second: repeated reads of one
    refresh count once, and refreshes first seen before the load (plus a
    quarter second) are left out."""
    import bench
    c = bench.ClockSampler()
    t0 = 100.0
    # (time, table counter, mean, min, max of the XCD clocks)
    c.samples = [(99.9, 1, 95.0, 90.0, 100.0), (100.1, 1, 95.0, 90.0, 100.0),
                 (100.2, 2, 1500.0, 1490.0, 1510.0), (100.5, 3, 1900.0, 1800.0, 2000.0),
                 (100.6, 3, 1900.0, 1800.0, 2000.0), (101.5, 4, 2000.0, 1950.0, 2050.0)]
    s = c.summary(t0)
    assert s["refreshes"] == 2 and s["mhz"] == 1950.0
    assert s["min_xcd_mhz"] == 1800.0 and s["max_xcd_mhz"] == 2050.0
    c.samples = c.samples[:2]
    assert c.summary(t0)["mhz"] is None

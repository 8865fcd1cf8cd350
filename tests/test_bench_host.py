"""CPU tests of bench.py's host logic: the HBM traffic figure is taken from the committed
counter record only for the kernel source and workload it was measured on, the committed
records agree with each other, and a request for more than one GPU is refused."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_is_used_only_for_its_kernel_source_and_workload(tmp_path, monkeypatch):
    b = _bench()
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(rec))
    assert b.traffic_per_launch("share_L128K_N8") is None  # no record
    rec.write_text(json.dumps({"kernel_sha": b.kernel_sha(), "workload": "share_L128K_N8",
                               "hbm_bytes_per_launch": 123}))
    assert b.traffic_per_launch("share_L128K_N8") == 123
    assert b.traffic_per_launch("share_L32K_N8") is None  # another workload
    rec.write_text(json.dumps({"kernel_sha": "0" * 16, "workload": "share_L128K_N8",
                               "hbm_bytes_per_launch": 123}))
    assert b.traffic_per_launch("share_L128K_N8") is None  # counters of another source
    rec.write_text("not json")
    assert b.traffic_per_launch("share_L128K_N8") is None


def test_committed_traffic_record_matches_the_headline_profile():
    """The counter record and the headline profile name the same kernel source."""
    b = _bench()
    with open(b.TRAFFIC_FILE) as f:
        rec = json.load(f)
    with open(os.path.join(ROOT, "profiles", "fwd_bf16_share_L128K_N8.md")) as f:
        prof = f.read()
    assert rec["workload"] == "share_L128K_N8"
    assert rec["kernel_sha"] in prof
    assert rec["hbm_bytes_per_launch"] > 0


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in (res.stdout + res.stderr)

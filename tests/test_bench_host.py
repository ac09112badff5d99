"""Host-side checks of bench.py (no GPU): the roofline arithmetic and the one-GPU contract."""
import subprocess
import sys
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_alu_roofline_constants():
    assert abs(bench.ALU_PEAK_TOPS - 256 * 4 * 16 * 2.4e9 / 1e12) < 1e-9
    assert bench.alu_ops_per_weight(0, False) == 4.0 and bench.alu_ops_per_weight(1, False) == 2.0
    assert bench.alu_ops_per_weight(0, True) == 3.0 and bench.alu_ops_per_weight(1, True) == 1.5


def test_algorithmic_bytes():
    # codes + x fp16 + y fp32 + scales fp16 + sign bits, for the 14336 -> 4096 K=3 layer
    assert bench.gemv_bytes(4096, 14336, 3) == 22020096 + 2 * 14336 + 4 * 4096 + 2 * 4096 + (14336 + 4096) // 8


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_recorded_traffic_only_for_the_sources_it_was_taken_on(monkeypatch):
    """profiles/traffic.json is tied to a hash of the kernel sources: the bench reports measured HBM
    traffic while that hash matches, and null once any kernel source has changed."""
    import json
    rec = json.load(open(bench.TRAFFIC_FILE))
    assert len(rec["csrc_sha"]) == 16 and bench.kernel_source_hash() == bench.kernel_source_hash()
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: rec["csrc_sha"])
    down = rec["workloads"]["2"]["down"]
    assert bench.recorded_traffic(2, "down") == down["hbm_bytes_per_launch"]
    assert down["hbm_bytes_per_launch"] == down["fetch_bytes_per_launch"] + down["write_bytes_per_launch"]
    assert bench.recorded_traffic(2, "no such launch") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.recorded_traffic(2, "down") is None

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

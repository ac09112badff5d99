"""Host-side checks of bench.py (no GPU): the roofline arithmetic and the one-GPU contract."""
import subprocess
import sys
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_is_the_largest_batch1_workload():
    """The bench's default workload is the 70B-shaped decoder layer (the largest batch-1 configuration),
    whose roofline is the HBM one: 8 TB/s."""
    from trellis_coded_gemv_amd import inputs
    assert bench.DEFAULT_WORKLOAD == 3 and inputs.WORKLOADS[3].name == "decoder70b_layer_k2"
    batch1 = [w for w in (1, 2, 3) if inputs.WORKLOADS[w].batch == 1]
    codes = {w: sum(m * n * k // 8 for m, n, k in inputs.WORKLOADS[w].tensors.values()) for w in batch1}
    assert max(codes, key=codes.get) == 3 and codes[3] == 213909504
    assert bench.HBM_PEAK_GBS == 8000.0


def test_cpu_baseline_uses_every_core_of_the_mask():
    """The oracle sample runs one worker process per core of the affinity mask (at most 16)."""
    rec, refs = bench.cpu_baseline(1, blocks_per_tensor=2, max_workers=16)
    assert rec["cores"] == min(len(os.sched_getaffinity(0)), 16)
    assert rec["affinity_cores"] == len(os.sched_getaffinity(0)) and rec["cpu_count"] == os.cpu_count()
    assert rec["kind"] == "oracle" and rec["value"] > 0 and len(refs) == 2


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
    key = sorted(rec["workloads"])[0]
    kern = sorted(rec["workloads"][key])[0]
    down = rec["workloads"][key][kern]
    assert bench.recorded_traffic(int(key.split("/")[0]), kern) == down["hbm_bytes_per_launch"]
    assert down["hbm_bytes_per_launch"] == down["fetch_bytes_per_launch"] + down["write_bytes_per_launch"]
    assert bench.recorded_traffic(2, "no such launch") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.recorded_traffic(int(key.split("/")[0]), kern) is None


def test_int8_mode_needs_mul1_and_keys_its_traffic(monkeypatch):
    """--int8 is the mul1 code's int8-activation form: refused with another code; its traffic record
    and its CPU baseline are the int8 form's own."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--int8", "--code", "0"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "--code 2" in r.stderr
    import json
    import numpy as np
    from oracle import gemv as ogemv
    from trellis_coded_gemv_amd import inputs
    rec = json.load(open(bench.TRAFFIC_FILE))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: rec["csrc_sha"])
    monkeypatch.setitem(bench.LAYER_FLAGS, "int8", True)
    if "3/code2/int8" in rec["workloads"]:
        assert bench.recorded_traffic(3, "gate_up", 2) == rec["workloads"]["3/code2/int8"]["gate_up"]["hbm_bytes_per_launch"]
    cpu, refs = bench.cpu_baseline(1, code_id=2, blocks_per_tensor=2, max_workers=2)
    assert "int8" in cpu["sample"]
    arr, x = bench.linear_inputs(inputs, inputs.WORKLOADS[1], 1, 2)["linear"]
    for (kind, name, b), y in refs.items():
        assert np.array_equal(y, ogemv.gemv_int8_rows(arr, x, np.arange(128 * b, 128 * b + 128)))


def test_context_codes_list():
    """The other codes measured beside the bench line: the line's own code and int8 forms that the
    workload cannot run are left out."""
    assert bench.context_codes("3,2i8,1", 0, False, 3) == [(3, False), (2, True), (1, False)]
    assert bench.context_codes("3,2i8,1", 3, False, 3) == [(2, True), (1, False)]
    assert bench.context_codes("3,2i8,1", 2, True, 3) == [(3, False), (1, False)]
    assert bench.context_codes("3,2i8", 0, False, 4) == [(3, False)]            # no int8 on the MFMA path
    assert bench.context_codes("", 0, False, 3) == []
    with pytest.raises(ValueError):
        bench.context_codes("5", 0, False, 3)

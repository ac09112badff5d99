"""Helpers shared by the GPU parity tests (device setup, tolerances, sampled rows)."""
import sys

import numpy as np
import pytest

from trellis_coded_gemv_amd import binding as tg

# Parity bar for fp32-accumulated outputs: max |y_gpu - y_ref| / max |y_ref| <= 1e-3
REL_TOL = 1e-3


def device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    tg.lib()            # raises if the HIP library is not built: no fallback
    return "cuda"


def say(*a):
    """Name the case before each GPU step (flushed), so a lost box still says what ran."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def rel_err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(y).all()
    return float(np.abs(y - ref).max() / np.abs(ref).max())


def sample_rows(m, seed=0, per_block=2):
    """Output indices to check against the oracle: per_block random outputs in every 128-output block
    (each block has its own split-K handoff; the oracle decodes only the tile rows it needs)."""
    rng = np.random.default_rng(seed)
    rows = [128 * b + np.sort(rng.choice(128, per_block, replace=False)) for b in range(m // 128)]
    return np.concatenate(rows)


def _refs_module():
    import importlib.util
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "make_full_size_refs.py")
    spec = importlib.util.spec_from_file_location("make_full_size_refs", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


_REFS = {}


def full_size_case(key):
    """(layer arrays, x bits, sampled output rows, checked activation rows or None, oracle y [rows x outputs])
    of a full-size case whose oracle outputs tests/golden/make_full_size_refs.py stored."""
    import json
    mod = _refs_module()
    if not _REFS:
        z = np.load(mod.OUT, allow_pickle=False)
        _REFS.update({k: z[k] for k in z.files})
    meta = json.loads(str(_REFS["meta"]))
    assert meta[key] == json.loads(json.dumps(mod.CASES[key])), f"stale reference for {key}: regenerate"
    arr, X, rows, pick = mod.case_inputs(key)
    assert np.array_equal(_REFS[key + "/rows"], rows)
    return arr, X, rows, pick, _REFS[key + "/y"]

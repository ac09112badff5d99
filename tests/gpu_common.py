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


def sample_rows(m, seed=0, blocks=3, per_block=16):
    """Output indices from the first, last and a random 128-block (the oracle decodes only those)."""
    rng = np.random.default_rng(seed)
    nb = m // 128
    chosen = sorted({0, nb - 1, int(rng.integers(0, nb))})[:blocks]
    rows = []
    for b in chosen:
        rows += list(128 * b + np.sort(rng.choice(128, per_block, replace=False)))
    return np.array(sorted(set(rows)))

"""The stored oracle outputs of the full-size GPU parity cases are current (no GPU).

tests/golden/make_full_size_refs.py writes them from oracle/ only; this check recomputes the
first 128-output block of a few cases with the oracle and compares bit for bit, so a change
of the oracle or of the seeded inputs without regenerating the file fails here."""
import json

import numpy as np
import pytest

from gpu_common import _refs_module
from oracle import gemv


@pytest.mark.parametrize("key", ["w3_k_c0", "w2_down_c1", "w4_gate_c1", "prefill_gate_m256_c0", "w3i8_k_c2", "w3f_v_c3"])
def test_first_block_matches_oracle(key):
    mod = _refs_module()
    z = np.load(mod.OUT, allow_pickle=False)
    assert json.loads(str(z["meta"]))[key] == json.loads(json.dumps(mod.CASES[key]))
    arr, X, rows, pick = mod.case_inputs(key)
    assert np.array_equal(z[key + "/rows"], rows)
    first = rows < 128
    if mod.CASES[key].get("int8"):
        y = gemv.gemv_int8_rows(arr, X, rows[first])[None, :]
    elif X.ndim == 1:
        y = gemv.gemv_rows(arr, X, rows[first])[None, :]
    else:
        y = gemv.gemm_rows(arr, X if pick is None else X[pick], rows[first])
    assert np.array_equal(y, z[key + "/y"][:, first])

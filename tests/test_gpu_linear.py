"""GPU parity for TrellisLinear: every dispatch path (one row, <= 64 rows, chunks of 64, prefill) against the oracle."""
import numpy as np
import pytest

from gpu_common import REL_TOL, device, rel_err, say
from oracle import gemv as ogemv
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(1024,), (1, 1024), (5, 1024), (2, 3, 1024), (100, 1024), (200, 1024)])
def test_trellis_linear_paths(shape):
    dev = device()
    import torch
    arr = inputs.make_layer(384, 1024, 2, 4100)
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    X = inputs.make_x(1024, 4100 + rows, rows=rows) if rows > 1 else inputs.make_x(1024, 4100)[None, :]
    lin = tg.TrellisLinear(tg.DeviceLayer(arr, dev))
    say("linear", shape, tg.TrellisLinear.path_for_rows(rows))
    y = lin(tg.fp16_tensor(X, dev).reshape(shape))
    torch.cuda.synchronize()
    assert tuple(y.shape) == shape[:-1] + (384,) and y.dtype == torch.float32
    y = y.reshape(rows, 384).cpu().numpy()
    pick = np.unique(np.linspace(0, rows - 1, min(rows, 9)).astype(int))
    ref = ogemv.gemm(arr, X[pick])
    for i, r in enumerate(pick):
        assert rel_err(y[r], ref[i]) <= REL_TOL, r
    y2 = lin(tg.fp16_tensor(X, dev).reshape(shape))        # workspaces kept: same bits again
    torch.cuda.synchronize()
    assert np.array_equal(y2.reshape(rows, 384).cpu().numpy(), y)

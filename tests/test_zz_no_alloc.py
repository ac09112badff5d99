"""GPU parity of trellis_gemv_noalloc (split-K state in the library's per-device array) against
trellis_gemv with a caller workspace: two calls in a row through the C ABI, the second on a
smaller layer, each equal to the workspace path (same kernels, same split counts) and within the
1e-3 bar of it; a layer beyond the array's limits is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest

from gpu_common import REL_TOL, device, rel_err, say
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu


def _noalloc(layer, x, y):
    import torch
    d = layer.desc()
    st = tg.lib().trellis_gemv_noalloc(ctypes.byref(d), x.data_ptr(), y.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
    return st


def test_noalloc_matches_workspace_path_twice():
    dev = device()
    import torch
    cases = [(1024, 4096, 3, 7001), (256, 2048, 2, 7002)]        # the second call: a smaller input
    for m, n, k, seed in cases:
        arr = inputs.make_layer(m, n, k, seed)
        L = tg.DeviceLayer(arr, dev)
        x = tg.fp16_tensor(inputs.make_x(n, seed), dev)
        say("noalloc", m, n, k)
        ref = tg.trellis_gemv(L, x, ws=tg.workspace(L, 1, dev))
        y = torch.full((m,), float("nan"), dtype=torch.float32, device=dev)
        assert _noalloc(L, x, y) == 0
        torch.cuda.synchronize()
        assert torch.equal(y, ref), (m, n, k)
        assert rel_err(y.cpu().numpy(), ref.cpu().numpy()) <= REL_TOL


def test_noalloc_refuses_layers_beyond_the_array():
    dev = device()
    import torch
    assert tg.lib().tg_noalloc_scratch_bytes() == 256 + 64 * 1024 + 1024 * 128 * 8
    arr = inputs.make_layer(32768, 4096, 2, 7003)
    L = tg.DeviceLayer(arr, dev, splits=16)                    # 256 blocks x 8 chunks = 2048 pairs
    x = tg.fp16_tensor(inputs.make_x(4096, 7003), dev)
    y = torch.full((32768,), 7.0, dtype=torch.float32, device=dev)
    say("noalloc refuses")
    assert _noalloc(L, x, y) == -5
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())

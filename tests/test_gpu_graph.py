"""Captured HIP graphs: several replays, with eager work between them, each equal to the eager result bit for bit."""
import numpy as np
import pytest

from gpu_common import device, say
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu


def _capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn(s)
    torch.cuda.synchronize()
    return g


def _replays(torch, g, out, ref, eager):
    for r in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        eager()                     # the program's own eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("code_id", [0, 1])
def test_graph_gemv_split_k(code_id):
    """Batch-1 GEMV with split-K (tickets and slots live in the workspace across replays)."""
    dev = device()
    import torch
    L = tg.DeviceLayer(inputs.make_layer(1024, 8192, 3, 5000 + code_id, code_id=code_id), dev)
    x = tg.fp16_tensor(inputs.make_x(8192, 5000), dev)
    ws = tg.workspace(L, 1, dev)
    say("graph gemv", code_id)
    ref = tg.trellis_gemv(L, x, ws=ws).clone()
    y = torch.empty_like(ref)
    g = _capture(torch, lambda s: tg.trellis_gemv(L, x, y, ws, s))
    _replays(torch, g, y, ref, lambda: tg.trellis_gemv(L, x, ws=ws))


def test_graph_gemm_small_and_moe_block():
    dev = device()
    import torch
    L = tg.DeviceLayer(inputs.make_layer(512, 4096, 2, 5100), dev)
    X = tg.fp16_tensor(inputs.make_x(4096, 5100, rows=16), dev)
    ws = tg.workspace(L, 16, dev)
    say("graph gemm_small")
    ref = tg.trellis_gemm_small(L, X, ws=ws).clone()
    Y = torch.empty_like(ref)
    g = _capture(torch, lambda s: tg.trellis_gemm_small(L, X, Y, ws, s))
    _replays(torch, g, Y, ref, lambda: tg.trellis_gemm_small(L, X, ws=ws))

    wl = inputs.MoEWorkload(experts=6, tokens=2)
    gu = tg.LayerTable([tg.DeviceLayer(wl.layer(e, w), dev) for e in range(6) for w in ("gate", "up")], dev)
    dn = tg.LayerTable([tg.DeviceLayer(wl.layer(e, "down"), dev) for e in range(6)], dev)
    sel = torch.tensor([5, 1, 3], dtype=torch.int32, device=dev)
    w = torch.tensor([0.5, 0.3, 0.2], dtype=torch.float32, device=dev)
    x = tg.fp16_tensor(inputs.make_x(wl.hidden, 5101), dev)
    mws = tg.moe_workspace(gu, dn, 3, dev)
    say("graph moe block")
    ref = tg.trellis_moe_block(gu, dn, sel, w, x, ws=mws).clone()
    y = torch.empty_like(ref)
    g = _capture(torch, lambda s: tg.trellis_moe_block(gu, dn, sel, w, x, y, mws, s))
    _replays(torch, g, y, ref, lambda: tg.trellis_moe_block(gu, dn, sel, w, x, ws=mws))
    assert np.isfinite(y.cpu().numpy()).all()

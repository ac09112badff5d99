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


@pytest.mark.parametrize("code_id,flags", [(0, 0), (2, tg.TG_FLAG_INT8_ACT)])
def test_graph_fused_launch(code_id, flags):
    """The fused launch of layers that share an input: its ticket counters and call-tagged slots live
    in the workspace across replays; the int8 form's quantiser runs inside the launch too."""
    dev = device()
    import torch
    n = 2048
    Ls = [tg.DeviceLayer(inputs.make_layer(m, n, 2, 5200 + m, code_id=code_id), dev, flags=flags)
          for m in (1024, 256, 256)]
    x = tg.fp16_tensor(inputs.make_x(n, 5200), dev)
    ws = tg.fused_workspace(Ls, dev)
    say("graph fused", code_id, flags)
    ref = torch.cat([y.clone() for y in tg.trellis_gemv_fused(Ls, x, ws=ws)])
    ys = [torch.empty(L.m, dtype=torch.float32, device=dev) for L in Ls]
    g = _capture(torch, lambda s: tg.trellis_gemv_fused(Ls, x, ys, ws, s))
    for r in range(3):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.cat(ys), ref), r
        tg.trellis_gemv_fused(Ls, x, ws=ws)     # eager work between replays, on the same workspace
        torch.cuda.synchronize()


def test_graph_noalloc_after_setup():
    """trellis_gemv_noalloc under capture once its device array is set up (the first call)."""
    dev = device()
    import ctypes
    import torch
    L = tg.DeviceLayer(inputs.make_layer(512, 4096, 2, 5300), dev)
    x = tg.fp16_tensor(inputs.make_x(4096, 5300), dev)
    d = L.desc()

    def call(y, s):
        assert tg.lib().trellis_gemv_noalloc(ctypes.byref(d), x.data_ptr(), y.data_ptr(), s.cuda_stream) == 0

    say("graph noalloc")
    ref = torch.empty(512, dtype=torch.float32, device=dev)
    call(ref, torch.cuda.current_stream())
    torch.cuda.synchronize()
    y = torch.empty_like(ref)
    g = _capture(torch, lambda s: call(y, s))
    _replays(torch, g, y, ref, lambda: call(torch.empty_like(ref), torch.cuda.current_stream()))


def test_graph_prefill():
    dev = device()
    import torch
    L = tg.DeviceLayer(inputs.make_layer(512, 2048, 3, 5400), dev)
    X = tg.fp16_tensor(inputs.make_x(2048, 5400, rows=600), dev)
    ws = tg.prefill_workspace(L, 600, dev)
    say("graph prefill")
    ref = tg.trellis_gemm_prefill(L, X, ws=ws).clone()
    Y = torch.empty_like(ref)
    g = _capture(torch, lambda s: tg.trellis_gemm_prefill(L, X, Y, ws, s))
    _replays(torch, g, Y, ref, lambda: tg.trellis_gemm_prefill(L, X, ws=ws))

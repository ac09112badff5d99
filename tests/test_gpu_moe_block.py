"""GPU parity for the mixture-of-experts block (gate/up -> silu * mul -> down -> router combine)."""
import numpy as np
import pytest

from gpu_common import REL_TOL, device, rel_err, say
from oracle import moe
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu


def _tables(dev, wl, code_id=0):
    gu = [wl.layer(e, w, code_id=code_id) for e in range(wl.experts) for w in ("gate", "up")]
    dn = [wl.layer(e, "down", code_id=code_id) for e in range(wl.experts)]
    return (gu, tg.LayerTable([tg.DeviceLayer(a, dev) for a in gu], dev),
            dn, tg.LayerTable([tg.DeviceLayer(a, dev) for a in dn], dev))


@pytest.mark.parametrize("token", [0, 1, 63])
def test_moe_block_workload_tokens(token):
    """128 experts (gate/up 2048->768, down 768->2048, K in {1,2,3}), top-8 with softmax router weights."""
    dev = device()
    import torch
    wl = inputs.CFG5
    gu, gut, dn, dnt = _tables(dev, wl)
    sel = wl.routing()[token]
    w = wl.router_weights()[token]
    x = inputs.make_x(wl.hidden, wl.seed, tensor=10_000 + token)
    say("moe block token", token, list(sel))
    y = tg.trellis_moe_block(gut, dnt, torch.from_numpy(sel).to(dev), torch.from_numpy(w).to(dev),
                             tg.fp16_tensor(x, dev))
    torch.cuda.synchronize()
    ref = moe.moe_block(gu, dn, sel, w, x)
    err = rel_err(y.cpu().numpy(), ref)
    say("rel err", err)
    assert err <= REL_TOL


def test_moe_block_pair_code_and_invalid_ids():
    """Pair-code experts; an out-of-range expert id contributes nothing (its weight is ignored)."""
    dev = device()
    import torch
    wl = inputs.MoEWorkload(experts=6, tokens=4)
    gu, gut, dn, dnt = _tables(dev, wl, code_id=1)
    sel = np.array([4, 99, 0, -1], np.int32)
    w = np.array([0.4, 0.3, 0.2, 0.1], np.float32)
    x = inputs.make_x(wl.hidden, 77)
    say("moe block pair code")
    ws = tg.moe_workspace(gut, dnt, 4, dev)
    # The workspace's last region holds the down projections, one row per selection; the rows of
    # the invalid selections are never written, so fill that region with NaN bit patterns first:
    # they must be dropped, not multiplied by a zero weight.
    ws[ws.numel() - 4 * wl.hidden * 4:] = 0xFF
    for _ in range(2):                      # the workspace is reused across calls
        y = tg.trellis_moe_block(gut, dnt, torch.from_numpy(sel).to(dev), torch.from_numpy(w).to(dev),
                                 tg.fp16_tensor(x, dev), ws=ws)
        torch.cuda.synchronize()
        ref = moe.moe_block(gu, dn, [4, 0], [0.4, 0.2], x)
        assert np.isfinite(y.cpu().numpy()).all()
        assert rel_err(y.cpu().numpy(), ref) <= REL_TOL


@pytest.mark.parametrize("code_id", [2, 3])
def test_moe_block_multiply_only_codes(code_id):
    """mul1 and MCG experts, each tensor with K drawn from {1, 2, 3} (paired windows at K = 1 and 2,
    the per-window form at K = 3)."""
    dev = device()
    import torch
    wl = inputs.MoEWorkload(experts=8, tokens=2)
    gu, gut, dn, dnt = _tables(dev, wl, code_id=code_id)
    sel = wl.routing()[1][:4].astype(np.int32)
    w = np.array([0.1, 0.2, 0.3, 0.4], np.float32)
    x = inputs.make_x(wl.hidden, 78 + code_id)
    say("moe block code", code_id, list(sel))
    y = tg.trellis_moe_block(gut, dnt, torch.from_numpy(sel).to(dev), torch.from_numpy(w).to(dev),
                             tg.fp16_tensor(x, dev))
    torch.cuda.synchronize()
    ref = moe.moe_block(gu, dn, sel, w, x)
    assert rel_err(y.cpu().numpy(), ref) <= REL_TOL

"""GPU parity: small-batch MFMA path and grouped (mixture-of-experts) GEMVs against the oracle."""
import numpy as np
import pytest

from gpu_common import REL_TOL, device, full_size_case, rel_err, say
from oracle import gemv as ogemv
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu


def _gemm(arr, X_bits, dev, flags=0):
    import torch
    L = tg.DeviceLayer(arr, dev, flags=flags)
    X = tg.fp16_tensor(X_bits, dev)
    Y = tg.trellis_gemm_small(L, X)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


@pytest.mark.parametrize("M", [1, 2, 15, 16, 17, 32, 33, 64])
def test_gemm_small_batches(M):
    dev = device()
    arr = inputs.make_layer(256, 512, 3, 3000 + M)
    X = inputs.make_x(512, 3000 + M, rows=M) if M > 1 else inputs.make_x(512, 3000 + M)[None, :]
    say("gemm_small M", M)
    Y = _gemm(arr, X, dev)
    ref = ogemv.gemm(arr, X)
    for r in range(M):
        assert rel_err(Y[r], ref[r]) <= REL_TOL, r


@pytest.mark.parametrize("flags", [0, tg.TG_FLAG_ROUND_WEIGHTS])
@pytest.mark.parametrize("k", range(1, 9))
def test_gemm_small_every_k(k, flags):
    dev = device()
    arr = inputs.make_layer(128, 384, k, 3100 + k)
    X = inputs.make_x(384, 3100 + k, rows=16)
    say("gemm_small k", k, flags)
    Y = _gemm(arr, X, dev, flags)
    ref = ogemv.gemm(arr, X)
    for r in range(16):
        assert rel_err(Y[r], ref[r]) <= REL_TOL, r


def test_gemm_small_matches_gemv_row_by_row():
    dev = device()
    import torch
    arr = inputs.make_layer(384, 1024, 2, 3200)
    X = inputs.make_x(1024, 3200, rows=5)
    Y = _gemm(arr, X, dev)
    L = tg.DeviceLayer(arr, dev)
    say("gemm vs gemv")
    for r in range(5):
        y = tg.trellis_gemv(L, tg.fp16_tensor(X[r], dev))
        torch.cuda.synchronize()
        assert rel_err(Y[r], y.cpu().numpy()) <= 2e-4


def test_gemm_small_config4_sampled():
    """Gate projection 8192->28672 at K=4 with 16 activation rows, in the bench's launch configuration."""
    dev = device()
    arr, X, rows, _, ref = full_size_case("w4_gate_c0")
    say("gemm_small cfg4")
    Y = _gemm(arr, X, dev)
    assert np.isfinite(Y).all()
    for r in range(X.shape[0]):
        assert rel_err(Y[r, rows], ref[r]) <= REL_TOL, r


def _moe_tables(dev, wl):
    """Two layer tables: gate/up (entry 2e + {0: gate, 1: up}) and down (entry e)."""
    gu = [wl.layer(e, w) for e in range(wl.experts) for w in ("gate", "up")]
    dn = [wl.layer(e, "down") for e in range(wl.experts)]
    return (gu, tg.LayerTable([tg.DeviceLayer(a, dev) for a in gu], dev),
            dn, tg.LayerTable([tg.DeviceLayer(a, dev) for a in dn], dev))


@pytest.mark.parametrize("token", [0, 1, 63])
def test_grouped_moe_config5(token):
    """Per token: one launch for the 16 gate/up GEMVs on a shared x, one for the 8 down GEMVs."""
    dev = device()
    import torch
    wl = inputs.CFG5
    gu, gu_table, dn, dn_table = _moe_tables(dev, wl)
    experts = wl.routing()[token]
    x = inputs.make_x(wl.hidden, wl.seed, tensor=10_000 + token)
    xd = inputs.make_x(wl.inter, wl.seed, tensor=20_000 + token, rows=wl.top_k)
    sel_gu = np.array([2 * int(e) + w for e in experts for w in (0, 1)], np.int32)
    sel_d = np.array([int(e) for e in experts], np.int32)
    say("grouped token", token, list(experts))
    Y1 = torch.zeros(len(sel_gu), wl.inter, dtype=torch.float32, device=dev)
    Y2 = torch.zeros(len(sel_d), wl.hidden, dtype=torch.float32, device=dev)
    tg.trellis_gemv_grouped(gu_table, torch.from_numpy(sel_gu).to(dev), tg.fp16_tensor(x, dev), 0, Y1, wl.inter)
    tg.trellis_gemv_grouped(dn_table, torch.from_numpy(sel_d).to(dev), tg.fp16_tensor(xd, dev), wl.inter, Y2,
                            wl.hidden)
    torch.cuda.synchronize()
    y1, y2 = Y1.cpu().numpy(), Y2.cpu().numpy()
    for e, li in enumerate(sel_gu):
        assert rel_err(y1[e], ogemv.gemv(gu[li], x)) <= REL_TOL, (e, li)
    for e, li in enumerate(sel_d):
        assert rel_err(y2[e], ogemv.gemv(dn[li], xd[e])) <= REL_TOL, (e, li)


def test_grouped_workspace_reuse():
    """A second call on the same workspace gives the same bits; the ticket counters end each call on a
    call boundary (low 16 bits zero)."""
    dev = device()
    import torch
    wl = inputs.CFG5
    _, _, dn, dn_table = _moe_tables(dev, wl)
    sel = torch.tensor([3, 77, 12, 100], dtype=torch.int32, device=dev)
    X = tg.fp16_tensor(inputs.make_x(wl.inter, 5, rows=4), dev)
    ws = tg.grouped_workspace(dn_table, 4, dev)
    say("grouped workspace reuse")
    Y1 = tg.trellis_gemv_grouped(dn_table, sel, X, wl.inter, torch.zeros(4, wl.hidden, device=dev), wl.hidden, ws)
    torch.cuda.synchronize()
    counters = 4 * (wl.hidden // 128) * 4                # one per selection and 128-output block
    assert int((ws[256: 256 + counters].view(torch.int32) & 0xFFFF).count_nonzero()) == 0
    Y2 = tg.trellis_gemv_grouped(dn_table, sel, X, wl.inter, torch.zeros(4, wl.hidden, device=dev), wl.hidden, ws)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


def test_grouped_out_of_range_selection_writes_nothing():
    dev = device()
    import torch
    wl = inputs.CFG5
    arrays, table, _, _ = _moe_tables(dev, wl)
    sel = torch.tensor([5, -1, 10_000, 7], dtype=torch.int32, device=dev)
    x = inputs.make_x(wl.hidden, 1)
    Y = torch.full((4, wl.inter), 7.0, dtype=torch.float32, device=dev)
    say("grouped out of range")
    tg.trellis_gemv_grouped(table, sel, tg.fp16_tensor(x, dev), 0, Y, wl.inter)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    assert (y[1] == 7.0).all() and (y[2] == 7.0).all()
    assert rel_err(y[0], ogemv.gemv(arrays[5], x)) <= REL_TOL
    assert rel_err(y[3], ogemv.gemv(arrays[7], x)) <= REL_TOL


@pytest.mark.parametrize("M,code_id", [(16, 0), (3, 0), (16, 1)])
def test_gemm_small_long_chunks(M, code_id):
    """One split over 6144 inputs: code 0 runs 16-wave workgroups (384 MFMA steps), the pair code
    8-wave ones; the full output is checked."""
    dev = device()
    arr = inputs.make_layer(128, 6144, 2, 3300 + M, code_id=code_id)
    X = inputs.make_x(6144, 3300 + M, rows=M)
    say("gemm_small long chunks", M, code_id)
    Y = _gemm(arr, X, dev)
    ref = ogemv.gemm(arr, X)
    for r in range(M):
        assert rel_err(Y[r], ref[r]) <= REL_TOL, r


@pytest.mark.parametrize("n_sel", [2, 8])
def test_grouped_mixed_shapes(n_sel):
    """One table mixing a 768x2048 and a 2048x768 layer (the launch's split count comes from the
    wider input; the narrower layer runs one chunk per 128-block), every output checked."""
    dev = device()
    import torch
    arrays = [inputs.make_layer(768, 2048, 2, 3400), inputs.make_layer(2048, 768, 3, 3401),
              inputs.make_layer(768, 2048, 1, 3402, code_id=1), inputs.make_layer(2048, 768, 2, 3403)]
    table = tg.LayerTable([tg.DeviceLayer(a, dev) for a in arrays], dev)
    sel = np.array([(1, 0, 3, 2)[e % 4] for e in range(n_sel)], np.int32)
    X = inputs.make_x(2048, 3404, rows=n_sel)
    say("grouped mixed shapes", n_sel, list(sel))
    Y = torch.full((n_sel, 2048), float("nan"), dtype=torch.float32, device=dev)
    tg.trellis_gemv_grouped(table, torch.from_numpy(sel).to(dev), tg.fp16_tensor(X, dev), 2048, Y, 2048)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    for e, li in enumerate(sel):
        m, n = arrays[li].m, arrays[li].n
        ref = ogemv.gemv(arrays[li], X[e, :n])      # selection e reads the first n inputs of its row
        assert rel_err(y[e, :m], ref) <= REL_TOL, (e, li)
        assert np.isnan(y[e, m:]).all()          # nothing past the layer's outputs is written

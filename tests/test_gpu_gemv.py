"""GPU parity: batch-1 trellis GEMV and the randomized Hadamard transform against the oracle."""

import numpy as np
import pytest

from gpu_common import REL_TOL, device, full_size_case, rel_err, sample_rows, say
from oracle import gemv as ogemv
from oracle import hadamard as ohad
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu

HDR = 256                                  # workspace header (status word) before the counter areas


def _run_gemv(arr, x_bits, dev, flags=0, ws=None, splits=0):
    torch = pytest.importorskip("torch")
    L = tg.DeviceLayer(arr, dev, flags=flags, splits=splits)
    x = tg.fp16_tensor(x_bits, dev)
    y = tg.trellis_gemv(L, x, ws=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("inverse", [False, True])
@pytest.mark.parametrize("n,rows", [(128, 1), (384, 3), (14336, 2)])
def test_rht_apply(n, rows, inverse):
    dev = device()
    rng = np.random.default_rng(n + rows)
    x = rng.standard_normal((rows, n)).astype(np.float16)
    sw = rng.integers(0, 1 << 32, n // 32, dtype=np.uint32)
    import torch
    say("rht", n, rows, inverse)
    out = tg.rht_apply(torch.from_numpy(x).to(dev), torch.from_numpy(sw.view(np.int32)).to(dev), inverse)
    xv = x.astype(np.float64)
    ref = ohad.rht_inverse(xv, sw) if inverse else ohad.rht_forward(xv, sw)
    assert np.abs(out.cpu().numpy() - ref).max() <= 1e-5 * np.abs(ref).max()


@pytest.mark.parametrize("flags", [0, tg.TG_FLAG_ROUND_WEIGHTS])
@pytest.mark.parametrize("k", range(1, 9))
@pytest.mark.parametrize("m,n", [(128, 128), (256, 384), (384, 256), (128, 1152)])
def test_gemv_small_shapes(k, m, n, flags):
    dev = device()
    arr = inputs.make_layer(m, n, k, 2000 + k, tensor=m * 7 + n)
    x = inputs.make_x(n, 2000 + k, tensor=m * 7 + n)
    say("gemv", m, n, k, flags)
    y = _run_gemv(arr, x, dev, flags)
    assert rel_err(y, ogemv.gemv(arr, x)) <= REL_TOL


def test_gemv_config1_full():
    dev = device()
    wl = inputs.CFG1
    m, n, k = wl.tensors["linear"]
    arr = inputs.make_layer(m, n, k, wl.seed)
    x = inputs.make_x(n, wl.seed)
    say("gemv cfg1")
    for flags in (0, tg.TG_FLAG_ROUND_WEIGHTS):
        y = _run_gemv(arr, x, dev, flags)
        err = rel_err(y, ogemv.gemv(arr, x))
        say("cfg1 flags", flags, "rel err", err)
        assert err <= REL_TOL


@pytest.mark.parametrize("cfg,tensor", [(2, "down"), (3, "q"), (3, "k"), (3, "v"), (3, "o"), (3, "gate"),
                                        (3, "up"), (3, "down")])
def test_gemv_config_sampled(cfg, tensor):
    """Full-size workload tensors in the launch configuration the bench times; oracle on sampled outputs."""
    dev = device()
    arr, x, rows, _, ref = full_size_case(f"w{cfg}_{tensor}_c0")
    say("gemv config", cfg, tensor, arr.m, arr.n, arr.k_bits)
    y = _run_gemv(arr, x, dev)
    assert np.isfinite(y).all()
    err = rel_err(y[rows], ref[0])
    say("rel err", err)
    assert err <= REL_TOL


def test_gemv_deterministic_and_workspace_reuse():
    dev = device()
    import torch
    arr = inputs.make_layer(1024, 4096, 3, 77)
    x = inputs.make_x(4096, 77)
    L = tg.DeviceLayer(arr, dev)
    ws = tg.workspace(L, 1, dev)
    xt = tg.fp16_tensor(x, dev)
    say("determinism")
    y1 = tg.trellis_gemv(L, xt, ws=ws).clone()
    y2 = tg.trellis_gemv(L, xt, ws=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    tickets = ws[HDR: HDR + 1024 // 128 * 4].view(torch.int32)
    assert ((tickets & 0xFFFF) == 0).all()              # ticket counters end each call at a call boundary
    rows = sample_rows(1024)
    assert rel_err(y1.cpu().numpy()[rows], ogemv.gemv_rows(arr, x, rows)) <= REL_TOL


@pytest.mark.parametrize("splits", ["1", "3", "7", "32"])
def test_gemv_split_counts(splits):
    """Every split count (forced through the layer's splits field) gives the same answer within tolerance."""
    dev = device()
    arr = inputs.make_layer(256, 4096, 2, 88)
    x = inputs.make_x(4096, 88)
    say("splits", splits)
    y = _run_gemv(arr, x, dev, splits=int(splits))
    assert rel_err(y, ogemv.gemv(arr, x)) <= REL_TOL


def test_gemv_edge_values():
    """Zero input gives zero output; an all-zero stream matches the oracle's closed-form case."""
    dev = device()
    arr = inputs.make_layer(256, 256, 2, 99)
    y = _run_gemv(arr, np.zeros(256, np.uint16), dev)
    assert (y == 0).all()
    arr.codes = np.zeros_like(arr.codes)
    x = inputs.make_x(256, 99)
    y = _run_gemv(arr, x, dev)
    assert rel_err(y, ogemv.gemv(arr, x)) <= REL_TOL


@pytest.mark.parametrize("splits", ["40", "64"])
def test_gemv_many_splits(splits):
    """More splits than one pass of the reducer covers (8 waves x 4 slots): chunks of one and two 128-blocks."""
    dev = device()
    arr = inputs.make_layer(256, 8192, 2, 89)
    x = inputs.make_x(8192, 89)
    say("many splits", splits)
    y = _run_gemv(arr, x, dev, splits=int(splits))
    assert rel_err(y, ogemv.gemv(arr, x)) <= REL_TOL



def test_gemv_slot_area_full_beside_small_batch():
    """A 32768 x 4096 layer with a forced 16 splits is held to the slot area's 2048 (block, split)
    pairs (256 blocks x 8 splits): its slots fill the area exactly. Batch-1 and 16-row calls then
    alternate on one buffer; each result equals the one on a fresh workspace, bit for bit, so the
    small-batch scratch and the full slot area do not overlap."""
    dev = device()
    import torch
    arr = inputs.make_layer(32768, 4096, 2, 96)
    L = tg.DeviceLayer(arr, dev, splits=16)
    x = inputs.make_x(4096, 96)
    xt = tg.fp16_tensor(x, dev)
    X = tg.fp16_tensor(inputs.make_x(4096, 97, rows=16), dev)
    say("slot area full", 32768, 4096)
    ref_v, ref_g = tg.trellis_gemv(L, xt), tg.trellis_gemm_small(L, X)
    ws = tg.workspace(L, 16, dev)
    for _ in range(2):
        assert torch.equal(tg.trellis_gemv(L, xt, ws=ws), ref_v)
        assert torch.equal(tg.trellis_gemm_small(L, X, ws=ws), ref_g)
    torch.cuda.synchronize()
    slots = ws[HDR + 2 * (1 << 22) // 128 * 4:].view(torch.int64)
    assert (((slots[: 2048 * 128] >> 32) & 0xFFFF) == 8).all()   # 8 splits in every pair's tag
    _, _, rows, _, ref = full_size_case("slots_32768x4096_c0")
    assert rel_err(ref_v.cpu().numpy()[rows], ref[0]) <= REL_TOL


def test_gemv_call_tags_wrap():
    """70,000 calls on one workspace: the 16-bit call number in the ticket counters and slot tags
    wraps (at 65,536 calls) without a stale partial ever being taken for a current one."""
    import torch
    dev = device()
    arr = inputs.make_layer(256, 4096, 2, 94)   # 2 blocks x 8 splits: every call hands over
    L = tg.DeviceLayer(arr, dev)
    x = tg.fp16_tensor(inputs.make_x(4096, 94), dev)
    ws = tg.workspace(L, 1, dev)
    y = torch.empty(256, dtype=torch.float32, device=dev)
    say("tag wrap: 70000 calls")
    ref = tg.trellis_gemv(L, x, ws=ws).clone()
    bad = torch.zeros((), dtype=torch.int32, device=dev)
    for i in range(70_000):
        tg.trellis_gemv(L, x, y, ws=ws)
        if i % 4096 == 4095 or i >= 65_530:
            bad += (~torch.eq(y, ref)).sum()
    torch.cuda.synchronize()
    assert int(bad) == 0
    tickets = ws[HDR: HDR + 2 * 4].view(torch.int32)
    assert ((tickets & 0xFFFF) == 0).all()


def test_workspace_shared_by_layers_and_paths():
    """One buffer serves two layers on both paths, its scratch first filled with ones (every split-K
    slot then carries a tag no call uses): each result equals the one computed on a fresh workspace,
    bit for bit; after every call the batch-1 ticket counters sit on a call boundary (low 16 bits
    zero) and the small-batch arrival counters are zero."""
    dev = device()
    import torch
    a_arr = inputs.make_layer(1024, 4096, 3, 90)
    b_arr = inputs.make_layer(512, 8192, 2, 91)
    A, B = tg.DeviceLayer(a_arr, dev), tg.DeviceLayer(b_arr, dev)
    xa, xb = tg.fp16_tensor(inputs.make_x(4096, 90), dev), tg.fp16_tensor(inputs.make_x(8192, 91), dev)
    Xa = tg.fp16_tensor(inputs.make_x(4096, 92, rows=16), dev)
    Xb = tg.fp16_tensor(inputs.make_x(8192, 93, rows=5), dev)
    size = max(tg.workspace(A, 16, dev).numel(), tg.workspace(B, 16, dev).numel())
    ws = torch.zeros(size, dtype=torch.uint8, device=dev)
    counters = HDR + 2 * (1 << 22) // 128 * 4  # end of the batch-1 and small-batch counter areas
    ws[counters:] = 0xFF
    say("shared workspace")
    ref = {"ga": tg.trellis_gemm_small(A, Xa), "vb": tg.trellis_gemv(B, xb),
           "gb": tg.trellis_gemm_small(B, Xb), "va": tg.trellis_gemv(A, xa)}
    calls = [("va", lambda: tg.trellis_gemv(A, xa, ws=ws)), ("ga", lambda: tg.trellis_gemm_small(A, Xa, ws=ws)),
             ("vb", lambda: tg.trellis_gemv(B, xb, ws=ws)), ("gb", lambda: tg.trellis_gemm_small(B, Xb, ws=ws)),
             ("va", lambda: tg.trellis_gemv(A, xa, ws=ws)), ("vb", lambda: tg.trellis_gemv(B, xb, ws=ws))]
    for name, call in calls:
        y = call()
        torch.cuda.synchronize()
        assert torch.equal(y, ref[name]), name
        half = (counters - HDR) // 2
        tickets = ws[HDR: HDR + half].view(torch.int32)
        assert ((tickets & 0xFFFF) == 0).all(), name
        assert (ws[HDR + half: counters] == 0).all(), name
    rows = sample_rows(512)
    assert rel_err(ref["vb"].cpu().numpy()[rows], ogemv.gemv_rows(b_arr, inputs.make_x(8192, 91), rows)) <= REL_TOL


def test_stale_slots_never_carry_the_expected_tag():
    """Two layers with 8 and 16 splits share one buffer, so a slot address belongs to different output
    blocks (and ticket counters) in turn. Read off the device around every batch-1 call: before it,
    no slot of the call's layout holds the tag the call waits for (its block's call number and its
    split count); after it, every slot of the layout holds exactly that tag, and y equals the result
    on a fresh workspace. The sequence is one where a tag of the call number alone would match a
    stale slot, which is asserted too, so the check does not rest on the reducer happening to read
    after the writers."""
    dev = device()
    import torch
    a_arr, b_arr = inputs.make_layer(1024, 4096, 3, 94), inputs.make_layer(512, 8192, 2, 95)
    A, B = tg.DeviceLayer(a_arr, dev), tg.DeviceLayer(b_arr, dev)
    xa, xb = tg.fp16_tensor(inputs.make_x(4096, 94), dev), tg.fp16_tensor(inputs.make_x(8192, 95), dev)
    ref = {"a": tg.trellis_gemv(A, xa), "b": tg.trellis_gemv(B, xb)}
    ws = torch.zeros(max(tg.workspace(A, 1, dev).numel(), tg.workspace(B, 1, dev).numel()),
                     dtype=torch.uint8, device=dev)
    counter_area = (1 << 22) // 128 * 4
    slot_off = HDR + 2 * counter_area            # the slot area follows the header and both counter areas
    say("stale slot tags")
    call_tag_alone_would_match = False
    for name in "ababa":
        L, x, ob = (A, xa, 8) if name == "a" else (B, xb, 4)
        pre = ws.clone()
        y = tg.trellis_gemv(L, x, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, ref[name]), name
        post_slots = ws[slot_off:].view(torch.int64)
        S = int((post_slots[0] >> 32) & 0xFFFF)   # the split count the call wrote
        assert S in (8, 16), S
        tickets = pre[HDR: HDR + counter_area].view(torch.int32)[:ob].to(torch.int64) & 0xFFFFFFFF
        expect = ((tickets & 0xFFFF0000) | S).view(ob, 1)
        n_slots = ob * S * 128
        after = ((post_slots[:n_slots] >> 32) & 0xFFFFFFFF).view(ob, S * 128)
        before = ((pre[slot_off:].view(torch.int64)[:n_slots] >> 32) & 0xFFFFFFFF).view(ob, S * 128)
        assert (after == expect).all(), name
        assert not (before == expect).any(), name
        old_rule = (tickets >> 16).view(ob, 1) + 1  # a tag of the call number + 1 alone
        call_tag_alone_would_match |= bool(((before >> 16) + 1 == old_rule).logical_and(before != 0).any())
    assert call_tag_alone_would_match


def test_workspace_status_word():
    """Calls that finish normally leave the status word at zero; the query reads the word and clears it."""
    dev = device()
    import torch
    arr = inputs.make_layer(256, 4096, 2, 98)
    L = tg.DeviceLayer(arr, dev)
    ws = tg.workspace(L, 1, dev)
    say("status word")
    tg.trellis_gemv(L, tg.fp16_tensor(inputs.make_x(4096, 98), dev), ws=ws)
    assert tg.workspace_status(ws) == 0
    ws[:4] = torch.tensor([tg.TG_STATUS_SPLITK_TIMEOUT, 0, 0, 0], dtype=torch.uint8, device=dev)
    assert tg.workspace_status(ws, clear=True) == tg.TG_STATUS_SPLITK_TIMEOUT
    assert tg.workspace_status(ws) == 0

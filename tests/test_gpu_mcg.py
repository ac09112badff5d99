"""GPU parity for MCG (code_id 3: the three-instruction code's generator with no additive
constant) against the oracle, through the C ABI: bit-exact decode, code table and encoder; the
products within 1e-3 of the largest output, as for code 0 (the default form adds the two fp16
halves inside the fp32 product, the rounded form rounds each weight to fp16 first, which the
oracle does). With K dividing 16 the batch-1 loops take two windows from one 32-bit span, so
K = 1, 2, 4, 8 run that form and K = 3, 5, 6, 7 the per-window one.
"""
import numpy as np
import pytest

from gpu_common import REL_TOL, device, full_size_case, rel_err, say
from oracle import code as ocode
from oracle import gemv as ogemv
from oracle import viterbi as ov
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu

MCG = 3
RW = tg.TG_FLAG_ROUND_WEIGHTS


def _layer(m, n, k, seed, tensor=0):
    return inputs.make_layer(m, n, k, seed, tensor=tensor, code_id=MCG)


def _gemv(arr, x_bits, dev, flags=0, splits=0):
    import torch
    L = tg.DeviceLayer(arr, dev, flags=flags, splits=splits)
    y = tg.trellis_gemv(L, tg.fp16_tensor(x_bits, dev))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_mcg_table_bit_exact():
    dev = device()
    say("mcg table")
    t = tg.code_table(dev, code_id=MCG).cpu().numpy().view(np.uint16)
    assert np.array_equal(t, ocode.mcg_table())


@pytest.mark.parametrize("k", range(1, 9))
@pytest.mark.parametrize("m,n", [(16, 16), (48, 32), (128, 384)])
def test_mcg_decode_bit_exact(k, m, n):
    dev = device()
    arr = _layer(m, n, k, 9300 + k, tensor=m + n)
    say("mcg decode", m, n, k)
    w = tg.trellis_decode(tg.DeviceLayer(arr, dev)).cpu().numpy().view(np.uint16)
    assert np.array_equal(w, ogemv.decode_layer(arr))


@pytest.mark.parametrize("k", [1, 2, 3])
def test_mcg_encode_matches_oracle(k):
    """The Viterbi encoder with MCG: words and costs equal to the oracle's, bit for bit."""
    dev = device()
    import torch
    tgt = np.random.default_rng(9400 + k).standard_normal((5, 256)).astype(np.float32)
    say("mcg encode", k)
    codes, err = tg.trellis_encode(torch.from_numpy(tgt).to(dev), k, MCG, 0.75)
    torch.cuda.synchronize()
    codes, err = codes.cpu().numpy().view(np.uint32), err.cpu().numpy()
    wvals = ov.code_values(MCG)
    for i in range(tgt.shape[0]):
        ref_words, ref_cost = ov.encode_tile(tgt[i], k, MCG, 0.75, wvals)
        assert np.array_equal(codes[i], ref_words), i
        assert err[i] == ref_cost, (i, err[i], ref_cost)


@pytest.mark.parametrize("flags", [0, RW])
@pytest.mark.parametrize("k", range(1, 9))
@pytest.mark.parametrize("m,n", [(128, 128), (256, 384), (128, 1152)])
def test_mcg_gemv_small_shapes(k, m, n, flags):
    dev = device()
    arr = _layer(m, n, k, 9500 + k, tensor=m * 7 + n)
    x = inputs.make_x(n, 9500 + k, tensor=m * 7 + n)
    say("mcg gemv", m, n, k, flags)
    assert rel_err(_gemv(arr, x, dev, flags), ogemv.gemv(arr, x)) <= REL_TOL


def test_mcg_one_hot_inputs():
    """One-hot inputs, unit scales, no signs: the transformed input of the hot block is +-1/sqrt(128)
    in every column, so every weight of that block enters with the same magnitude and no
    cancellation between columns can hide a wrong weight from either half of a span."""
    dev = device()
    import torch
    m, n, k = 128, 128, 2
    arr = _layer(m, n, k, 9550)
    arr.scales = np.full(m, 0x3C00, np.uint16)
    arr.sign_in = np.zeros_like(arr.sign_in)
    arr.sign_out = np.zeros_like(arr.sign_out)
    L = tg.DeviceLayer(arr, dev)
    say("mcg columns")
    for c in (0, 5, 8, 13, 127):
        x = np.zeros(n, np.float16)
        x[c] = 1.0
        y = tg.trellis_gemv(L, tg.fp16_tensor(x.view(np.uint16), dev))
        torch.cuda.synchronize()
        assert rel_err(y.cpu().numpy(), ogemv.gemv(arr, x.view(np.uint16))) <= REL_TOL, c


@pytest.mark.parametrize("splits", [1, 3, 7, 32])
def test_mcg_gemv_split_counts(splits):
    dev = device()
    arr = _layer(256, 4096, 2, 9600)
    x = inputs.make_x(4096, 9600)
    say("mcg splits", splits)
    assert rel_err(_gemv(arr, x, dev, 0, splits), ogemv.gemv(arr, x)) <= REL_TOL


@pytest.mark.parametrize("flags", [0, RW])
@pytest.mark.parametrize("splits", [0, 7, 37])
def test_mcg_fused_small_layers(flags, splits):
    dev = device()
    import torch
    n = 1024
    arrays = [_layer(m, n, 2, 9700 + m) for m in (512, 128, 256)]
    x = inputs.make_x(n, 9701)
    layers = [tg.DeviceLayer(a, dev, flags=flags, splits=splits) for a in arrays]
    say("mcg fused small", flags, splits)
    ys = tg.trellis_gemv_fused(layers, tg.fp16_tensor(x, dev))
    torch.cuda.synchronize()
    for a, y in zip(arrays, ys):
        assert rel_err(y.cpu().numpy(), ogemv.gemv(a, x)) <= REL_TOL


@pytest.mark.parametrize("group", [("q", "k", "v"), ("gate", "up")])
def test_mcg_decoder_layer_fused_full_size(group):
    """The 70B-shaped layer's fused launches with MCG, as the bench runs them: two outputs of every
    128-output block of every layer against stored oracle outputs."""
    dev = device()
    import torch
    cases = [full_size_case(f"w3f_{name}_c3") for name in group]
    x = cases[0][1]
    assert all(np.array_equal(c[1], x) for c in cases)
    layers = [tg.DeviceLayer(c[0], dev) for c in cases]
    say("mcg fused full size", group)
    ys = tg.trellis_gemv_fused(layers, tg.fp16_tensor(x, dev))
    torch.cuda.synchronize()
    for (arr, _, rows, _, ref), y in zip(cases, ys):
        y = y.cpu().numpy()
        assert np.isfinite(y).all()
        err = rel_err(y[rows], ref[0])
        say("rel err", err)
        assert err <= REL_TOL


@pytest.mark.parametrize("name", ["o", "down", "k"])
def test_mcg_gemv_full_size(name):
    dev = device()
    arr, x, rows, _, ref = full_size_case(f"w3_{name}_c3")
    say("mcg gemv full size", name)
    err = rel_err(_gemv(arr, x, dev)[rows], ref[0])
    say("rel err", err)
    assert err <= REL_TOL


@pytest.mark.parametrize("flags", [0, RW])
@pytest.mark.parametrize("M,k", [(1, 3), (16, 3), (33, 3), (16, 2), (5, 4), (16, 4), (40, 8), (16, 1)])
def test_mcg_gemm_small(M, k, flags):
    """K = 2, 4, 8 run the paired windows and the paired x~ column order; K = 1, 3 the plain form."""
    dev = device()
    import torch
    arr = _layer(256, 512, k, 9800 + M + 10 * k)
    X = inputs.make_x(512, 9800 + M, rows=M) if M > 1 else inputs.make_x(512, 9800 + M)[None, :]
    say("mcg gemm M", M, k, flags)
    Y = tg.trellis_gemm_small(tg.DeviceLayer(arr, dev, flags=flags), tg.fp16_tensor(X, dev))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    ref = ogemv.gemm(arr, X)
    for r in range(M):
        assert rel_err(Y[r], ref[r]) <= REL_TOL, r


def test_mcg_prefill():
    dev = device()
    import torch
    arr = _layer(384, 1024, 2, 9900)
    X = inputs.make_x(1024, 9900, rows=80)
    say("mcg prefill")
    Y = tg.trellis_gemm_prefill(tg.DeviceLayer(arr, dev), tg.fp16_tensor(X, dev))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    for r in (0, 41, 79):
        assert rel_err(Y[r], ogemv.gemv(arr, X[r])) <= REL_TOL, r


def test_grouped_all_four_codes():
    """A grouped launch over a table whose experts use all four codes."""
    dev = device()
    import torch
    wl = inputs.CFG5
    arrays = [wl.layer(e, "gate", code_id=e % 4) for e in range(12)]
    table = tg.LayerTable([tg.DeviceLayer(a, dev) for a in arrays], dev)
    sel = np.array([3, 7, 0, 11, 6, 9, 1], np.int32)
    X = inputs.make_x(wl.hidden, 9950, rows=len(sel))
    Y = torch.zeros(len(sel), wl.inter, dtype=torch.float32, device=dev)
    say("grouped four codes")
    tg.trellis_gemv_grouped(table, torch.from_numpy(sel).to(dev), tg.fp16_tensor(X, dev), wl.hidden, Y, wl.inter)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    for e, li in enumerate(sel):
        assert rel_err(y[e], ogemv.gemv(arrays[li], X[e])) <= REL_TOL, (e, li)


def test_mcg_decode_ceiling_runs():
    dev = device()
    import torch
    say("mcg ceiling")
    out = tg.decode_ceiling(2, MCG, 8, 16)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("code_id", [2, 3])
def test_multiply_only_codes_gemm_small_config4(code_id):
    """The 28672 x 8192 gate projection at K=4 with 16 rows (paired windows and column order) for
    mul1 and MCG: two outputs of every 128-output block of every row against stored oracle outputs."""
    dev = device()
    import torch
    arr, X, rows, _, ref = full_size_case(f"w4_gate_c{code_id}")
    say("gemm_small cfg4", code_id)
    Y = tg.trellis_gemm_small(tg.DeviceLayer(arr, dev), tg.fp16_tensor(X, dev))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    assert np.isfinite(Y).all()
    for r in range(X.shape[0]):
        assert rel_err(Y[r, rows], ref[r]) <= REL_TOL, r


@pytest.mark.parametrize("k", [4, 6, 8])
def test_mcg_encode_high_rates_consistent(k):
    """Wider steps (the oracle's search is too slow here): each stored stream decodes, through the
    oracle's walk and code, to the error the encoder reports, and the error falls with the rate."""
    dev = device()
    import torch
    tgt = np.random.default_rng(9450 + k).standard_normal((3, 256)).astype(np.float32)
    say("mcg encode", k)
    codes, err = tg.trellis_encode(torch.from_numpy(tgt).to(dev), k, MCG, 0.75)
    torch.cuda.synchronize()
    codes, err = codes.cpu().numpy().view(np.uint32), err.cpu().numpy()
    for i in range(3):
        recomputed = ov.tile_errors(codes[i], tgt[i], k, MCG, 0.75)
        assert abs(recomputed - float(err[i])) <= 1e-4 * max(recomputed, 1e-3), i
    assert float(err.mean()) / 256 < {4: 0.012, 6: 0.004, 8: 0.003}[k]

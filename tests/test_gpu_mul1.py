"""GPU parity for mul1 (code_id 2) and its int8-activation form (TG_FLAG_INT8_ACT) against the oracle,
through the C ABI.

The weights of mul1 are exact in fp16 and, in the int8 form, the quantised input and every integer
product are exact on both sides (the oracle's quantiser and the kernels' take the same decisions from
exact float64 values), so only fp32 accumulation and the fp32 output transform round: the bar here is
2e-5 of the largest output, tight enough that one quantisation step taken differently in one input
element fails it. The small-batch and prefill paths round x~ to fp16 and keep the 1e-3 bar.
"""
import ctypes

import numpy as np
import pytest

from gpu_common import REL_TOL, device, full_size_case, rel_err, say
from oracle import code as ocode
from oracle import gemv as ogemv
from oracle import viterbi as ov
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu

MUL1 = 2
I8 = tg.TG_FLAG_INT8_ACT
TIGHT = 2e-5


def _layer(m, n, k, seed, tensor=0):
    return inputs.make_layer(m, n, k, seed, tensor=tensor, code_id=MUL1)


def _ref(arr, x, flags):
    return ogemv.gemv_int8(arr, x) if flags & I8 else ogemv.gemv(arr, x)


def _gemv(arr, x_bits, dev, flags=0, splits=0):
    import torch
    L = tg.DeviceLayer(arr, dev, flags=flags, splits=splits)
    y = tg.trellis_gemv(L, tg.fp16_tensor(x_bits, dev))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_mul1_table_bit_exact():
    dev = device()
    say("mul1 table")
    t = tg.code_table(dev, code_id=MUL1).cpu().numpy().view(np.uint16)
    assert np.array_equal(t, ocode.mul1_table())


@pytest.mark.parametrize("k", range(1, 9))
@pytest.mark.parametrize("m,n", [(16, 16), (48, 32), (128, 384)])
def test_mul1_decode_bit_exact(k, m, n):
    dev = device()
    arr = _layer(m, n, k, 8000 + k, tensor=m + n)
    say("mul1 decode", m, n, k)
    w = tg.trellis_decode(tg.DeviceLayer(arr, dev)).cpu().numpy().view(np.uint16)
    assert np.array_equal(w, ogemv.decode_layer(arr))


@pytest.mark.parametrize("k", [1, 2, 3])
def test_mul1_encode_matches_oracle(k):
    """The Viterbi encoder with the mul1 code: words and costs equal to the oracle's, bit for bit."""
    dev = device()
    import torch
    tgt = np.random.default_rng(8100 + k).standard_normal((5, 256)).astype(np.float32)
    say("mul1 encode", k)
    codes, err = tg.trellis_encode(torch.from_numpy(tgt).to(dev), k, MUL1, 0.9)
    torch.cuda.synchronize()
    codes, err = codes.cpu().numpy().view(np.uint32), err.cpu().numpy()
    wvals = ov.code_values(MUL1)
    for i in range(tgt.shape[0]):
        ref_words, ref_cost = ov.encode_tile(tgt[i], k, MUL1, 0.9, wvals)
        assert np.array_equal(codes[i], ref_words), i
        assert err[i] == ref_cost, (i, err[i], ref_cost)


@pytest.mark.parametrize("flags", [0, I8])
@pytest.mark.parametrize("k", range(1, 9))
@pytest.mark.parametrize("m,n", [(128, 128), (256, 384), (128, 1152)])
def test_mul1_gemv_small_shapes(k, m, n, flags):
    dev = device()
    arr = _layer(m, n, k, 8200 + k, tensor=m * 7 + n)
    x = inputs.make_x(n, 8200 + k, tensor=m * 7 + n)
    say("mul1 gemv", m, n, k, flags)
    assert rel_err(_gemv(arr, x, dev, flags), _ref(arr, x, flags)) <= TIGHT


@pytest.mark.parametrize("flags", [0, I8])
@pytest.mark.parametrize("splits", [1, 3, 7, 32])
def test_mul1_gemv_split_counts(flags, splits):
    """Chunks of one, a few and many 128-blocks; a ragged last chunk (odd block counts per chunk)."""
    dev = device()
    arr = _layer(256, 4096, 2, 8300)
    x = inputs.make_x(4096, 8300)
    say("mul1 splits", flags, splits)
    assert rel_err(_gemv(arr, x, dev, flags, splits), _ref(arr, x, flags)) <= TIGHT


def test_int8_lossless_equals_plain_product():
    """Small integer inputs quantise without loss (every block's scale is a power of two at most 1):
    the int8 form then equals the plain product of the oracle."""
    dev = device()
    n = 1024
    arr = _layer(256, n, 3, 8400)
    rng = np.random.default_rng(8400)
    x = np.zeros(n, np.float16)
    idx = rng.choice(n, 60, replace=False)
    x[idx] = rng.integers(-2, 3, 60)
    q, e = ogemv.quantize_rotated(arr, x.view(np.uint16))
    assert (e <= 0).all()
    say("int8 lossless")
    y = _gemv(arr, x.view(np.uint16), dev, I8)
    assert rel_err(y, ogemv.gemv(arr, x.view(np.uint16))) <= TIGHT


def test_int8_wide_range_and_zero_blocks():
    """Inputs spanning the whole fp16 range (the transform is exact only in float64), an all-zero
    block, and an all-zero vector (zero output)."""
    dev = device()
    n = 768
    arr = _layer(256, n, 4, 8500)
    rng = np.random.default_rng(8500)
    mag = np.exp2(rng.integers(-24, 15, n).astype(np.float64)) * rng.choice([-1, 1], n)
    x = (mag * rng.uniform(1, 2, n)).astype(np.float16)
    x[256:384] = 0
    say("int8 wide range")
    xb = x.view(np.uint16)
    assert rel_err(_gemv(arr, xb, dev, I8), ogemv.gemv_int8(arr, xb)) <= TIGHT
    assert (_gemv(arr, np.zeros(n, np.uint16), dev, I8) == 0).all()


def test_int8_noalloc_equals_workspace_path():
    dev = device()
    import torch
    arr = _layer(512, 2048, 2, 8600)
    L = tg.DeviceLayer(arr, dev, flags=I8)
    x = tg.fp16_tensor(inputs.make_x(2048, 8600), dev)
    say("int8 noalloc")
    ref = tg.trellis_gemv(L, x)
    y = torch.full((512,), float("nan"), dtype=torch.float32, device=dev)
    d = L.desc()
    assert tg.lib().trellis_gemv_noalloc(ctypes.byref(d), x.data_ptr(), y.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(y, ref)


@pytest.mark.parametrize("flags", [0, I8])
@pytest.mark.parametrize("splits", [0, 7, 37])
def test_mul1_fused_small_layers(flags, splits):
    dev = device()
    import torch
    n = 1024
    arrays = [_layer(m, n, 3, 8700 + m) for m in (512, 128, 256)]
    x = inputs.make_x(n, 8701)
    layers = [tg.DeviceLayer(a, dev, flags=flags, splits=splits) for a in arrays]
    say("mul1 fused small", flags, splits)
    ys = tg.trellis_gemv_fused(layers, tg.fp16_tensor(x, dev))
    torch.cuda.synchronize()
    for a, y in zip(arrays, ys):
        assert rel_err(y.cpu().numpy(), _ref(a, x, flags)) <= TIGHT


@pytest.mark.parametrize("n", [128, 384, 16384])
def test_int8_fused_widths(n):
    """A single block, an odd block count, and the widest input (two transform passes)."""
    dev = device()
    import torch
    arrays = [_layer(256, n, 2, 8800 + n), _layer(128, n, 2, 8801 + n)]
    x = inputs.make_x(n, 8802 + n)
    layers = [tg.DeviceLayer(a, dev, flags=I8, splits=13) for a in arrays]
    say("int8 fused widths", n)
    ys = tg.trellis_gemv_fused(layers, tg.fp16_tensor(x, dev))
    torch.cuda.synchronize()
    for a, y in zip(arrays, ys):
        assert rel_err(y.cpu().numpy(), ogemv.gemv_int8(a, x)) <= TIGHT


@pytest.mark.parametrize("group", [("q", "k", "v"), ("gate", "up")])
def test_int8_decoder_layer_fused_full_size(group):
    """The 70B-shaped layer's fused launches with mul1 and int8 activations, as the bench runs them:
    two outputs of every 128-output block of every layer against stored oracle outputs."""
    dev = device()
    import torch
    cases = [full_size_case(f"w3i8_{name}_c2") for name in group]
    x = cases[0][1]
    assert all(np.array_equal(c[1], x) for c in cases)
    layers = [tg.DeviceLayer(c[0], dev, flags=I8) for c in cases]
    say("int8 fused full size", group)
    ys = tg.trellis_gemv_fused(layers, tg.fp16_tensor(x, dev))
    torch.cuda.synchronize()
    for (arr, _, rows, _, ref), y in zip(cases, ys):
        err = rel_err(y.cpu().numpy()[rows], ref[0])
        say("rel err", err)
        assert err <= TIGHT


@pytest.mark.parametrize("key,flags", [("w3i8_o_c2", I8), ("w3i8_down_c2", I8), ("w3_down_c2", 0)])
def test_mul1_gemv_full_size(key, flags):
    dev = device()
    arr, x, rows, _, ref = full_size_case(key)
    say("mul1 gemv full size", key)
    err = rel_err(_gemv(arr, x, dev, flags)[rows], ref[0])
    say("rel err", err)
    assert err <= TIGHT


@pytest.mark.parametrize("M,k", [(1, 3), (16, 3), (33, 3), (16, 2), (7, 4), (16, 4), (48, 8)])
def test_mul1_gemm_small(M, k):
    """K = 2, 4, 8 run the paired windows and the paired x~ column order; K = 3 the plain form."""
    dev = device()
    import torch
    arr = _layer(256, 512, k, 8900 + M + 10 * k)
    X = inputs.make_x(512, 8900 + M, rows=M) if M > 1 else inputs.make_x(512, 8900 + M)[None, :]
    say("mul1 gemm M", M, k)
    Y = tg.trellis_gemm_small(tg.DeviceLayer(arr, dev), tg.fp16_tensor(X, dev))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    ref = ogemv.gemm(arr, X)
    for r in range(M):
        assert rel_err(Y[r], ref[r]) <= REL_TOL, r


def test_mul1_prefill():
    dev = device()
    import torch
    arr = _layer(384, 1024, 2, 9000)
    X = inputs.make_x(1024, 9000, rows=80)
    say("mul1 prefill")
    Y = tg.trellis_gemm_prefill(tg.DeviceLayer(arr, dev), tg.fp16_tensor(X, dev))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    for r in (0, 41, 79):
        assert rel_err(Y[r], ogemv.gemv(arr, X[r])) <= REL_TOL, r


def test_mul1_grouped_mixed_codes():
    """A grouped launch over a table whose experts use all three codes."""
    dev = device()
    import torch
    wl = inputs.CFG5
    arrays = [wl.layer(e, "gate", code_id=e % 3) for e in range(12)]
    table = tg.LayerTable([tg.DeviceLayer(a, dev) for a in arrays], dev)
    sel = np.array([2, 5, 0, 11, 7, 4], np.int32)
    X = inputs.make_x(wl.hidden, 9100, rows=len(sel))
    Y = torch.zeros(len(sel), wl.inter, dtype=torch.float32, device=dev)
    say("mul1 grouped mixed")
    tg.trellis_gemv_grouped(table, torch.from_numpy(sel).to(dev), tg.fp16_tensor(X, dev), wl.hidden, Y, wl.inter)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    for e, li in enumerate(sel):
        assert rel_err(y[e], ogemv.gemv(arrays[li], X[e])) <= REL_TOL, (e, li)


@pytest.mark.parametrize("flags", [0, I8])
def test_mul1_decode_ceiling_runs(flags):
    dev = device()
    import torch
    say("mul1 ceiling", flags)
    out = tg.decode_ceiling(2, MUL1, 8, 16, flags=flags)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("k", [4, 6, 8])
def test_mul1_encode_high_rates_consistent(k):
    """Wider steps (the oracle's search is too slow here): each stored stream decodes, through the
    oracle's walk and code, to the error the encoder reports, and the error falls with the rate."""
    dev = device()
    import torch
    tgt = np.random.default_rng(8150 + k).standard_normal((3, 256)).astype(np.float32)
    say("mul1 encode", k)
    codes, err = tg.trellis_encode(torch.from_numpy(tgt).to(dev), k, MUL1, 0.9)
    torch.cuda.synchronize()
    codes, err = codes.cpu().numpy().view(np.uint32), err.cpu().numpy()
    for i in range(3):
        recomputed = ov.tile_errors(codes[i], tgt[i], k, MUL1, 0.9)
        assert abs(recomputed - float(err[i])) <= 1e-4 * max(recomputed, 1e-3), i
    assert float(err.mean()) / 256 < {4: 0.012, 6: 0.004, 8: 0.003}[k]

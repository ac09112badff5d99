"""GPU parity for the pair code (code_id 1: one trellis state per two weights) against the oracle."""
import numpy as np
import pytest

from gpu_common import REL_TOL, device, full_size_case, rel_err, say
from oracle import code as ocode
from oracle import gemv as ogemv
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu

PAIR = 1


def _layer(m, n, k, seed, tensor=0):
    return inputs.make_layer(m, n, k, seed, tensor=tensor, code_id=PAIR)


def _gemv(arr, x_bits, dev, flags=0, splits=0):
    import torch
    L = tg.DeviceLayer(arr, dev, flags=flags, splits=splits)
    y = tg.trellis_gemv(L, tg.fp16_tensor(x_bits, dev))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _gemm(arr, X_bits, dev, flags=0):
    import torch
    L = tg.DeviceLayer(arr, dev, flags=flags)
    Y = tg.trellis_gemm_small(L, tg.fp16_tensor(X_bits, dev))
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def test_pair_code_table_bit_exact():
    dev = device()
    say("pair code table")
    t = tg.code_table(dev, code_id=PAIR).cpu().numpy().view(np.uint16)
    assert np.array_equal(t, ocode.pair_table())


@pytest.mark.parametrize("k", range(1, 9))
@pytest.mark.parametrize("m,n", [(16, 16), (48, 32), (128, 384), (256, 128)])
def test_pair_decode_bit_exact(k, m, n):
    dev = device()
    arr = _layer(m, n, k, 4000 + k, tensor=m + n)
    say("pair decode", m, n, k)
    w = tg.trellis_decode(tg.DeviceLayer(arr, dev)).cpu().numpy().view(np.uint16)
    assert np.array_equal(w, ogemv.decode_layer(arr))


def test_pair_decode_full_size_sampled():
    dev = device()
    m, n, k = inputs.CFG2.tensors["down"]
    arr = _layer(m, n, k, inputs.CFG2.seed)
    say("pair decode 4096x14336 K3")
    w = tg.trellis_decode(tg.DeviceLayer(arr, dev)).cpu().numpy().view(np.uint16)
    trows = [0, 117, m // 16 - 1]
    got = np.concatenate([w[16 * r:16 * r + 16] for r in trows])
    assert np.array_equal(got, ogemv.decode_layer(arr, trows))


@pytest.mark.parametrize("flags", [0, tg.TG_FLAG_ROUND_WEIGHTS])
@pytest.mark.parametrize("k", range(1, 9))
@pytest.mark.parametrize("m,n", [(128, 128), (256, 384), (128, 1152)])
def test_pair_gemv_small_shapes(k, m, n, flags):
    dev = device()
    arr = _layer(m, n, k, 4100 + k, tensor=m * 7 + n)
    x = inputs.make_x(n, 4100 + k, tensor=m * 7 + n)
    say("pair gemv", m, n, k, flags)
    assert rel_err(_gemv(arr, x, dev, flags), ogemv.gemv(arr, x)) <= REL_TOL


@pytest.mark.parametrize("cfg,tensor", [(2, "down"), (3, "k"), (3, "gate"), (3, "down")])
def test_pair_gemv_full_size_sampled(cfg, tensor):
    """Full-size workload shapes in the bench's launch configuration, oracle on sampled outputs."""
    dev = device()
    arr, x, rows, _, ref = full_size_case(f"w{cfg}_{tensor}_c1")
    say("pair gemv config", cfg, tensor, arr.m, arr.n, arr.k_bits)
    y = _gemv(arr, x, dev)
    err = rel_err(y[rows], ref[0])
    say("rel err", err)
    assert err <= REL_TOL


@pytest.mark.parametrize("splits", ["1", "3", "7"])
def test_pair_gemv_split_counts(splits):
    dev = device()
    arr = _layer(256, 4096, 2, 4200)
    x = inputs.make_x(4096, 4200)
    say("pair splits", splits)
    assert rel_err(_gemv(arr, x, dev, splits=int(splits)), ogemv.gemv(arr, x)) <= REL_TOL


def test_pair_gemv_zero_stream_and_zero_input():
    dev = device()
    arr = _layer(256, 384, 3, 4300)
    say("pair zero cases")
    assert (_gemv(arr, np.zeros(384, np.uint16), dev) == 0).all()
    arr.codes = np.zeros_like(arr.codes)
    x = inputs.make_x(384, 4300)
    assert rel_err(_gemv(arr, x, dev), ogemv.gemv(arr, x)) <= REL_TOL


@pytest.mark.parametrize("M", [1, 2, 16, 17, 33, 64])
def test_pair_gemm_small_batches(M):
    dev = device()
    arr = _layer(256, 512, 3, 4400 + M)
    X = inputs.make_x(512, 4400 + M, rows=M) if M > 1 else inputs.make_x(512, 4400 + M)[None, :]
    say("pair gemm M", M)
    Y = _gemm(arr, X, dev)
    ref = ogemv.gemm(arr, X)
    for r in range(M):
        assert rel_err(Y[r], ref[r]) <= REL_TOL, r


@pytest.mark.parametrize("flags", [0, tg.TG_FLAG_ROUND_WEIGHTS])
@pytest.mark.parametrize("k", range(1, 9))
@pytest.mark.parametrize("n", [128, 384])
def test_pair_gemm_small_every_k(k, n, flags):
    dev = device()
    arr = _layer(128, n, k, 4500 + k)
    X = inputs.make_x(n, 4500 + k, rows=16)
    say("pair gemm k", k, n, flags)
    Y = _gemm(arr, X, dev, flags)
    ref = ogemv.gemm(arr, X)
    for r in range(16):
        assert rel_err(Y[r], ref[r]) <= REL_TOL, r


def test_pair_gemm_full_size_sampled():
    """Gate projection 8192->28672 at K=4, 16 activation rows, pair code."""
    dev = device()
    arr, X, rows, _, ref = full_size_case("w4_gate_c1")
    say("pair gemm 28672x8192 K4 M16")
    Y = _gemm(arr, X, dev)
    for r in range(X.shape[0]):
        assert rel_err(Y[r, rows], ref[r]) <= REL_TOL, r


def test_pair_grouped_mixed_codes():
    """One grouped launch over a table whose experts alternate between code 0 and the pair code."""
    dev = device()
    import torch
    wl = inputs.CFG5
    arrays = [wl.layer(e, "gate", code_id=e % 2) for e in range(16)]
    table = tg.LayerTable([tg.DeviceLayer(a, dev) for a in arrays], dev)
    sel = np.array([3, 0, 7, 12, 9, 4], np.int32)
    X = inputs.make_x(wl.hidden, 4600, rows=len(sel))
    Y = torch.zeros(len(sel), wl.inter, dtype=torch.float32, device=dev)
    say("pair grouped mixed")
    tg.trellis_gemv_grouped(table, torch.from_numpy(sel).to(dev), tg.fp16_tensor(X, dev), wl.hidden, Y, wl.inter)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    for e, li in enumerate(sel):
        assert rel_err(y[e], ogemv.gemv(arrays[li], X[e])) <= REL_TOL, (e, li)

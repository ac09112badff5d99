"""GPU parity for the prefill path (each weight decoded once per 512 rows straight into the matrix-core
operands, rounded to fp16) against the oracle."""
import numpy as np
import pytest

from gpu_common import REL_TOL, device, full_size_case, rel_err, say
from oracle import gemv as ogemv
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu


def _prefill(arr, X_bits, dev):
    import torch
    L = tg.DeviceLayer(arr, dev)
    Y = tg.trellis_gemm_prefill(L, tg.fp16_tensor(X_bits, dev))
    torch.cuda.synchronize()
    return Y.cpu().numpy()


@pytest.mark.parametrize("k", range(1, 9))
@pytest.mark.parametrize("code_id", [0, 1, 2])
def test_prefill_every_k(k, code_id):
    dev = device()
    arr = inputs.make_layer(256, 384, k, 5000 + k, code_id=code_id)
    X = inputs.make_x(384, 5000 + k, rows=40)
    say("prefill k", k, code_id)
    Y = _prefill(arr, X, dev)
    ref = ogemv.gemm(arr, X)
    for r in range(40):
        assert rel_err(Y[r], ref[r]) <= REL_TOL, r


@pytest.mark.parametrize("M", [1, 2, 17, 64, 129, 512, 513, 1100])
def test_prefill_batch_sizes(M):
    """Up to and past one workgroup's 512 rows (a second and third row chunk, the last one partial)."""
    dev = device()
    arr = inputs.make_layer(384, 1152, 3, 5100 + M)
    X = inputs.make_x(1152, 5100 + M, rows=M) if M > 1 else inputs.make_x(1152, 5100 + M)[None, :]
    say("prefill M", M)
    Y = _prefill(arr, X, dev)
    ref = ogemv.gemm(arr, X)
    for r in range(M):
        assert rel_err(Y[r], ref[r]) <= REL_TOL, r


def test_prefill_decoded_weights_match_the_decode_hook():
    """A unit input row picks out one column of W_eff: the prefill's in-register decode checked
    column by column against the oracle's effective matrix on a small layer."""
    dev = device()
    arr = inputs.make_layer(128, 256, 2, 5200)
    X = np.zeros((3, 256), np.float16)
    for r, j in enumerate((0, 77, 255)):
        X[r, j] = 1.0
    say("prefill impulses")
    Y = _prefill(arr, X.view(np.uint16), dev)
    Weff = ogemv.effective_matrix(arr)
    for r, j in enumerate((0, 77, 255)):
        assert rel_err(Y[r], Weff[:, j]) <= REL_TOL, j


def test_prefill_full_size_sampled():
    """Gate projection 8192 -> 28672 at K=4 with 256 rows: sampled outputs against the oracle."""
    dev = device()
    arr, X, rows, pick, ref = full_size_case("prefill_gate_m256_c0")
    say("prefill 28672x8192 K4 M256")
    Y = _prefill(arr, X, dev)
    assert np.isfinite(Y).all()
    for i, r in enumerate(pick):
        assert rel_err(Y[r, rows], ref[i]) <= REL_TOL, r


def test_prefill_matches_mfma_path_with_rounded_weights():
    """Same rounded weights, same fp16 inputs: the two batched paths differ only in summation order."""
    dev = device()
    import torch
    arr = inputs.make_layer(256, 2048, 2, 5300)
    X = inputs.make_x(2048, 5300, rows=16)
    Yp = _prefill(arr, X, dev)
    L = tg.DeviceLayer(arr, dev, flags=tg.TG_FLAG_ROUND_WEIGHTS)
    Ys = tg.trellis_gemm_small(L, tg.fp16_tensor(X, dev))
    torch.cuda.synchronize()
    for r in range(16):
        assert rel_err(Yp[r], Ys.cpu().numpy()[r]) <= 1e-5, r


@pytest.mark.parametrize("m,n,M", [(384, 1152, 129), (28672, 8192, 512)])
def test_prefill_deterministic_and_strided(m, n, M):
    """Two calls give bit-identical outputs (no atomics: each output is summed by one wave in a
    fixed order), and an output row stride wider than m leaves the gap columns untouched."""
    import torch
    dev = device()
    arr = inputs.make_layer(m, n, 2, 5300 + M)
    X = tg.fp16_tensor(inputs.make_x(n, 5300 + M, rows=M), dev)
    L = tg.DeviceLayer(arr, dev)
    say("prefill determinism", m, n, M)
    Y1 = tg.trellis_gemm_prefill(L, X).clone()
    Y2 = tg.trellis_gemm_prefill(L, X).clone()
    wide = torch.full((M, m + 128), 7.0, dtype=torch.float32, device=dev)
    tg.trellis_gemm_prefill(L, X, Y=wide[:, :m])
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
    assert torch.isfinite(Y1).all()
    assert torch.equal(wide[:, m:], torch.full_like(wide[:, m:], 7.0))
    assert rel_err(wide[:, :m].cpu().numpy(), Y1.cpu().numpy()) <= REL_TOL

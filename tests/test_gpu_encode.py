"""GPU parity for the tail-biting Viterbi encoder against the oracle.

Floating point decides the stored bits here, so the oracle takes every
decision in the kernel's precision (float32, same operation order, same
tie-breaks): codes and squared errors must match bit for bit.
"""
import numpy as np
import pytest

from gpu_common import device, say
from oracle import trellis
from oracle import viterbi as ov
from trellis_coded_gemv_amd import binding as tg
from trellis_coded_gemv_amd import inputs

pytestmark = pytest.mark.gpu

SCALE = {0: 0.75, 1: 0.8}


def _targets(n_tiles, seed):
    return np.random.default_rng(seed).standard_normal((n_tiles, 256)).astype(np.float32)


def _encode(tgt, k, code_id, scale):
    import torch
    t = torch.from_numpy(tgt).to(device())
    codes, err = tg.trellis_encode(t, k, code_id, scale)
    torch.cuda.synchronize()
    return codes.cpu().numpy().view(np.uint32), err.cpu().numpy()


@pytest.mark.parametrize("code_id,k", [(0, 1), (0, 2), (0, 3), (0, 4), (1, 1), (1, 2)])
def test_encode_bit_exact_against_oracle(code_id, k):
    tgt = _targets(2, 7000 + 10 * code_id + k)
    say("encode parity", code_id, k)
    codes, err = _encode(tgt, k, code_id, SCALE[code_id])
    wvals = ov.code_values(code_id)
    for i in range(tgt.shape[0]):
        ref_words, ref_cost = ov.encode_tile(tgt[i], k, code_id, SCALE[code_id], wvals)
        assert np.array_equal(codes[i], ref_words), i
        assert err[i] == ref_cost, (i, err[i], ref_cost)


@pytest.mark.parametrize("code_id,k", [(0, 5), (0, 6), (0, 7), (0, 8), (1, 3), (1, 4)])
def test_encode_high_rates_consistent(code_id, k):
    """Wider steps (oracle too slow here): the stored stream decodes to the reported error, which
    falls with the bit width, and every stream is a closed circle by construction of the format."""
    tgt = _targets(3, 7100 + 10 * code_id + k)
    say("encode consistency", code_id, k)
    codes, err = _encode(tgt, k, code_id, SCALE[code_id])
    for i in range(3):
        recomputed = ov.tile_errors(codes[i], tgt[i], k, code_id, SCALE[code_id])
        assert abs(recomputed - float(err[i])) <= 1e-4 * max(recomputed, 1e-3), i
    assert float(err.mean()) / 256 < {5: 0.004, 6: 0.0015, 7: 0.0008, 8: 0.0008, 3: 0.03, 4: 0.012}[k]


@pytest.mark.parametrize("code_id,k", [(0, 2), (0, 5), (1, 2)])
def test_encode_representable_targets_exactly(code_id, k):
    """Targets equal to the decoded weights of a stored tile are encoded with zero error."""
    words = inputs.make_layer(16, 64, k, 7200 + k).codes.reshape(4, 8 * k)
    v = 2 if code_id == 1 else 1
    wvals = ov.code_values(code_id)
    tgt = np.stack([wvals[trellis.walk_states(trellis.stream_bits(w, k), k, v)].reshape(-1) for w in words])
    say("encode exact", code_id, k)
    codes, err = _encode(tgt.astype(np.float32), k, code_id, 1.0)
    assert (err == 0).all()
    for i in range(4):
        assert ov.tile_errors(codes[i], tgt[i], k, code_id, 1.0) == 0.0


def test_encode_many_tiles_gaussian_mse():
    """More tiles than workgroups (the persistent tile loop); two bits on a Gaussian source.
    The pages quote about 0.069 for their trellis code and 1/16 for the rate-distortion bound."""
    tgt = _targets(600, 7300)
    say("encode 600 tiles K=2")
    codes, err = _encode(tgt, 2, 0, SCALE[0])
    mse = float(err.astype(np.float64).sum() / tgt.size)
    say("mse", mse)
    assert 0.060 < mse < 0.070
    wvals = ov.code_values(0)
    for i in (0, 257, 599):
        ref_words, ref_cost = ov.encode_tile(tgt[i], 2, 0, SCALE[0], wvals)
        assert np.array_equal(codes[i], ref_words) and err[i] == ref_cost, i

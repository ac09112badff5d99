"""Pins for the oracle's tail-biting Viterbi encoder (no GPU).

Small trellises (an L=6 bit window) are searched exhaustively: the open
Viterbi pass must reach the exact minimum over every linear bit string, and
the two-pass tail-biting result must be a closed circle no better than the
exact optimum over every circle. On the real 16-bit trellis, sequences the
code can represent exactly must be encoded with zero error, and the mean
squared error on a Gaussian source at two bits must sit near the pages' figure.
"""
import itertools

import numpy as np
import pytest

from oracle import trellis
from oracle import viterbi as ov
from trellis_coded_gemv_amd import inputs


def _windows_linear(bits, L, b, T):
    """States of a linear (open) bit string: S_t = bits[b t : b t + L]."""
    out = []
    for t in range(T):
        s = 0
        for i in range(L):
            s = (s << 1) | int(bits[b * t + i])
        out.append(s)
    return out


def _windows_circle(bits, L, b, T):
    n = len(bits)
    return [int("".join(str(int(bits[(b * t + i) % n])) for i in range(L)), 2) for t in range(T)]


def _cost(states, wvals, alpha, targets):
    w = wvals[np.asarray(states)].astype(np.float64)
    return float(((alpha * w - targets.astype(np.float64)) ** 2).sum())


@pytest.mark.parametrize("b,T,seed", [(2, 6, 0), (1, 10, 1), (3, 4, 2)])
def test_open_viterbi_equals_exhaustive_search(b, T, seed):
    """[TQ] Part seven: the dynamic programme finds the best path -- checked against every bit string."""
    L = 6
    rng = np.random.default_rng(seed)
    wvals = rng.standard_normal(1 << L).astype(np.float32)
    targets = rng.standard_normal(T).astype(np.float32)
    nbits = L + b * (T - 1)
    best = min(_cost(_windows_linear(bits, L, b, T), wvals, 1.0, targets)
               for bits in itertools.product((0, 1), repeat=nbits))
    states, cost = ov.viterbi(wvals, 1.0, targets, L, b)
    assert abs(float(cost) - best) <= 1e-5 * max(best, 1e-3)
    assert abs(_cost(states, wvals, 1.0, targets) - best) <= 1e-5 * max(best, 1e-3)
    nxt = np.asarray(states[1:])
    assert ((nxt >> b) == (np.asarray(states[:-1]) & ((1 << (L - b)) - 1))).all()   # a valid path


@pytest.mark.parametrize("L,b,T,seed", [(6, 2, 6, 0), (6, 1, 12, 1), (5, 1, 16, 2)])
def test_constrained_pass_over_every_start_equals_exhaustive_circle_search(L, b, T, seed):
    """The second pass's constraint ([TQ] Part eight: start and end with the same bits) is exactly
    the tail-biting condition: its minimum over every start state is the best of all circles."""
    rng = np.random.default_rng(seed)
    wvals = rng.standard_normal(1 << L).astype(np.float32)
    targets = rng.standard_normal(T).astype(np.float32)
    exact = min(_cost(_windows_circle(bits, L, b, T), wvals, 1.0, targets)
                for bits in itertools.product((0, 1), repeat=b * T))
    best = min(float(ov.viterbi(wvals, 1.0, targets, L, b, start=s0, end_low=s0 >> b)[1]) for s0 in range(1 << L))
    assert abs(best - exact) <= 1e-5 * max(exact, 1e-3)


def test_two_pass_tail_biting_closes_the_circle_near_the_optimum():
    """The two-pass result is a closed circle whose decoded error is the reported cost; it is never
    better than the exhaustive optimum and, over twenty random cases, within 20% of it on average."""
    L, b, T = 5, 1, 16
    idx = (b * np.arange(T)[:, None] + np.arange(L)[None, :]) % (b * T)
    circles = np.array(list(itertools.product((0, 1), repeat=b * T)), dtype=np.int64)
    all_states = (circles[:, idx] << np.arange(L - 1, -1, -1)).sum(-1)          # [2^(bT), T]
    ratios = []
    for seed in range(20):
        rng = np.random.default_rng(100 + seed)
        wvals = rng.standard_normal(1 << L).astype(np.float32)
        targets = rng.standard_normal(T).astype(np.float32)
        exact = ((wvals[all_states].astype(np.float64) - targets) ** 2).sum(-1).min()
        states, cost = ov.encode_tail_biting(wvals, 1.0, targets, L, b)
        s = np.asarray(states)
        assert ((np.roll(s, -1) >> b) == (s & ((1 << (L - b)) - 1))).all()   # S_{T-1} steps back to S_0
        got = _cost(states, wvals, 1.0, targets)
        assert abs(got - float(cost)) <= 1e-5 * max(got, 1e-3)
        assert got >= exact - 1e-9
        ratios.append(got / exact)
    assert np.mean(ratios) < 1.2, ratios


@pytest.mark.parametrize("code_id,k", [(0, 2), (0, 3), (1, 1), (2, 2), (3, 2)])
def test_representable_sequence_is_encoded_exactly(code_id, k):
    """Targets that are the decoded weights of some stored tile are reached with zero error."""
    words = inputs.make_layer(16, 16, k, 55 + k).codes
    v = 2 if code_id == 1 else 1
    s = trellis.walk_states(trellis.stream_bits(words, k), k, v)
    wvals = ov.code_values(code_id)
    target = wvals[s].reshape(-1).astype(np.float32)
    out, cost = ov.encode_tile(target, k, code_id, 1.0, wvals)
    assert float(cost) == 0.0
    assert ov.tile_errors(out, target, k, code_id, 1.0) == 0.0


def test_packing_round_trip():
    rng = np.random.default_rng(3)
    words = rng.integers(0, 1 << 32, 24, dtype=np.uint32)
    assert np.array_equal(ov.pack_bits(trellis.stream_bits(words, 3)), words)


def test_gaussian_source_two_bits_mse():
    """[TQ] Part nine: at two bits on a Gaussian source the rate-distortion bound is 1/16 and the
    trellis with a computed code gets about 0.069; Lloyd-Max scalar quantization gets about 0.118.
    Sixteen N(0,1) tiles, code 0 at its reconstruction scale 0.75."""
    rng = np.random.default_rng(2024)
    wvals = ov.code_values(0)
    mse = np.mean([float(ov.encode_tile(rng.standard_normal(256).astype(np.float32), 2, 0, 0.75, wvals)[1]) / 256
                   for _ in range(16)])
    assert 0.055 < mse < 0.075, mse


def test_gaussian_source_two_bits_mse_mul1():
    """The same measurement with the mul1 code (code_id 2) at its reconstruction scale 0.9:
    a little above the three-instruction code, well under Lloyd-Max's 0.118 ([TQ] Part nine)."""
    rng = np.random.default_rng(2024)
    wvals = ov.code_values(2)
    assert wvals.shape == (1 << 16,) and (wvals * 32 == np.rint(wvals * 32)).all()
    mse = np.mean([float(ov.encode_tile(rng.standard_normal(256).astype(np.float32), 2, 2, 0.9, wvals)[1]) / 256
                   for _ in range(16)])
    assert 0.062 < mse < 0.080, mse


def test_gaussian_source_two_bits_mse_mcg():
    """The same measurement with MCG (code_id 3, the multiply-only generator) at scale 0.75:
    the trellis figure [TQ] Part nine gives for computed codes (about 0.069), far under
    Lloyd-Max's 0.118."""
    rng = np.random.default_rng(2024)
    wvals = ov.code_values(3)
    mse = np.mean([float(ov.encode_tile(rng.standard_normal(256).astype(np.float32), 2, 3, 0.75, wvals)[1]) / 256
                   for _ in range(16)])
    assert 0.055 < mse < 0.075, mse

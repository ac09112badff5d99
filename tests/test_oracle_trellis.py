"""Pins for the oracle's bitshift trellis (no GPU)."""
import numpy as np
import pytest

from conftest import golden_rows
from oracle import trellis


def _tile_from_bits(bits):
    """Pack a 256K-long MSB-first bit list into 8K uint32 words (test-side packing)."""
    bits = np.asarray(bits, dtype=np.uint64).reshape(-1, 32)
    weights = (1 << (31 - np.arange(32))).astype(np.uint64)
    return (bits * weights).sum(axis=1).astype(np.uint32)


def _random_tiles(k, count, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << 32, size=(count, 8 * k), dtype=np.uint32)


def test_figure_transitions():
    """The L=12, b=2 state-shift figure and the transition equation (Deep Dive, Section 3)."""
    for L, b, s, u, s1 in golden_rows("trellis_figure_l12_b2.txt"):
        got = trellis.step(int(s, 2), int(u, 2), int(b), int(L))
        assert int(got) == int(s1, 2)


def test_weight100_reads_bit200():
    """Random access at bit K*t (lecture, Part eight): single-bit streams."""
    for k, p, t, expect in golden_rows("weight100_bit200.txt"):
        k, p, t = int(k), int(p), int(t)
        bits = np.zeros(256 * k, dtype=np.uint8)
        bits[p] = 1
        words = _tile_from_bits(bits)
        b = trellis.stream_bits(words, k)
        assert (b == bits).all()
        assert int(trellis.walk_states(b, k)[t]) == int(expect, 16)
        assert int(trellis.window_states(b, k)[t]) == int(expect, 16)


@pytest.mark.parametrize("k", range(1, 9))
def test_walk_equals_random_access(k):
    b = trellis.stream_bits(_random_tiles(k, 64, 10 + k), k)
    assert (trellis.walk_states(b, k) == trellis.window_states(b, k)).all()


@pytest.mark.parametrize("k", range(1, 9))
def test_states_rebuild_stream_and_close_circle(k):
    b = trellis.stream_bits(_random_tiles(k, 64, 20 + k), k)
    s = trellis.walk_states(b, k)
    assert (trellis.stream_from_states(s, k) == b).all()
    assert trellis.closes_circle(s, b, k).all()
    assert trellis.is_valid_path(s, k).all()
    assert s.min() >= 0 and s.max() < 1 << 16


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_corrupted_paths_rejected(k):
    b = trellis.stream_bits(_random_tiles(k, 16, 30 + k), k)
    s = trellis.walk_states(b, k)
    rng = np.random.default_rng(k)
    for i in range(16):
        bad = s[i].copy()
        t = rng.integers(0, 256)
        bad[t] ^= 1 << int(rng.integers(0, 16 - k))     # flip a bit shared with a neighbour
        assert not trellis.is_valid_path(bad, k)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_every_single_bit_lands_where_the_window_puts_it(k):
    """Exhaustive brute force: one set bit at p shows up in state t iff d=(p-Kt) mod 256K <= 15, as bit 15-d."""
    nb = 256 * k
    t = np.arange(256)
    for p in range(nb):
        bits = np.zeros(nb, dtype=np.uint8)
        bits[p] = 1
        s = trellis.walk_states(trellis.stream_bits(_tile_from_bits(bits), k), k)
        d = (p - k * t) % nb
        expect = np.where(d <= 15, 1 << (15 - np.minimum(d, 15)), 0)
        assert (s == expect).all(), p


@pytest.mark.parametrize("k", [1, 2, 5])
def test_constant_streams(k):
    zeros = trellis.walk_states(trellis.stream_bits(np.zeros(8 * k, np.uint32), k), k)
    ones = trellis.walk_states(trellis.stream_bits(np.full(8 * k, 0xFFFFFFFF, np.uint32), k), k)
    assert (zeros == 0).all() and (ones == 0xFFFF).all()


def test_word_bit_order_msb_first():
    """Reading: stream bit p is bit 31 - p%32 of word p//32."""
    w = np.zeros(16, np.uint32)
    w[0] = 0x80000000
    w[1] = 0x00000001
    b = trellis.stream_bits(w, 2)
    assert b[0] == 1 and b[63] == 1 and b.sum() == 2


def test_layer_addressing_tile_row_major():
    """Tile (R, C) is tile R*(n/16)+C; inside it t = 16 r + c (readings)."""
    m, n, k = 48, 64, 1
    codes = np.zeros((m // 16) * (n // 16) * 8 * k, np.uint32)
    T = trellis.tile_index(2, 1, n)
    codes[T * 8 * k:(T + 1) * 8 * k] = 0xFFFFFFFF
    mat = trellis.states_to_matrix(trellis.layer_states(codes, m, n, k))
    assert mat.shape == (m, n)
    assert (mat[32:48, 16:32] == 0xFFFF).all()
    mask = np.ones_like(mat, dtype=bool)
    mask[32:48, 16:32] = False
    assert (mat[mask] == 0).all()
    # a single bit at stream position K*t of tile (0,0) is the MSB of state t -> row t//16, col t%16
    codes[:] = 0
    t = 37
    codes[(k * t) // 32] = np.uint32(1 << (31 - (k * t) % 32))
    mat = trellis.states_to_matrix(trellis.layer_states(codes, m, n, k))
    assert mat[t // 16, t % 16] == 0x8000


@pytest.mark.parametrize("k", range(1, 9))
def test_pair_steps_walk_equals_random_access(k):
    """V=2 steps ([DD] Section 3: b*V bits per V-dimensional step): 128 states of 2K new bits."""
    b = trellis.stream_bits(_random_tiles(k, 32, 40 + k), k)
    s = trellis.walk_states(b, k, v=2)
    assert s.shape[-1] == 128
    assert (s == trellis.window_states(b, k, v=2)).all()
    assert (trellis.stream_from_states(s, k, v=2) == b).all()
    assert trellis.closes_circle(s, b, k, v=2).all()
    assert trellis.is_valid_path(s, k, v=2).all()


def test_pair_steps_weight100_reads_bit200():
    """With V=2 at K=2, weights 100 and 101 share state 50, whose window starts at bit 200."""
    bits = np.zeros(512, dtype=np.uint8)
    bits[200] = 1
    s = trellis.walk_states(trellis.stream_bits(_tile_from_bits(bits), 2), 2, v=2)
    assert s[50] == 0x8000 and s[49] == 0x0800 and s[51] == 0


@pytest.mark.parametrize("k", [1, 2, 3])
def test_pair_steps_single_bits(k):
    nb = 256 * k
    tau = np.arange(128)
    for p in range(nb):
        bits = np.zeros(nb, dtype=np.uint8)
        bits[p] = 1
        s = trellis.walk_states(trellis.stream_bits(_tile_from_bits(bits), k), k, v=2)
        d = (p - 2 * k * tau) % nb
        assert (s == np.where(d <= 15, 1 << (15 - np.minimum(d, 15)), 0)).all(), p


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_broken_circle_rejected(k):
    """closes_circle is False once the first state, or a low bit of the last state, no longer
    follows the circle (the tail-biting closure of the lecture, Part eight)."""
    b = trellis.stream_bits(_random_tiles(k, 32, 50 + k), k)
    s = trellis.walk_states(b, k)
    assert trellis.closes_circle(s, b, k).all()
    first = s.copy()
    first[:, 0] ^= 1                    # the bit the closing step shifts in last
    assert not trellis.closes_circle(first, b, k).any()
    last = s.copy()
    last[:, -1] ^= 1 << (15 - k) if k < 16 else 1   # a bit the closing step keeps
    assert not trellis.closes_circle(last, b, k).any()
    tail = b.copy()
    tail[:, 15] ^= 1                    # the stream's bit 15 closes the circle
    assert not trellis.closes_circle(s, tail, k).any()

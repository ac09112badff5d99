"""Bitshift trellis: tile bitstreams, states, tail-biting walk (test infrastructure).

Definitions followed:
  * [DD] Section 3, transition equation: S_{t+1} = ((S_t << b) AND (2^L - 1)) OR u_t,
    with b new bits entering at the least significant end; the L=12, b=2
    figure shows the oldest bits leaving at the top.
  * [TQ] Part eight: the state is a 16-bit window into the tile's bit string;
    weight t's window starts at bit K*t (weight one hundred -> bit two hundred
    at two bits); a 16x16 tile of 256 weights is one sequence; the tail-biting
    trellis treats the stream as a circle, so a sequence holds exactly 256*K
    bits and the final windows wrap onto the first bits.

V-dimensional steps ([DD] Section 3, "b*V bits per V-dimensional sub-vector"):
with V=2 a sequence of 256 weights is 128 steps of two weights; each step
shifts 2K bits and the state of step tau starts at stream bit 2K*tau.

Readings where the pages are silent:
  * the first stream bit of a window is the state's most significant bit;
  * stream bit p of a tile is bit (31 - p mod 32) of 32-bit word p // 32
    (MSB-first inside little-endian words); a tile is 8*K words;
  * sequence position t = 16*r + c for row r, column c of the tile;
  * tiles are stored tile-row-major: tile (R, C) is tile number R*(n/16) + C.

Pins (tests/test_oracle_trellis.py): walk == random-access windows; the
stream rebuilt from the states' top K bits equals the input; closure of the
circle; every state pair is a valid trellis edge and corrupted sequences are
rejected; single-bit streams land exactly where the window definition puts
them (including the page's weight-100 / bit-200 statement); the L=12, b=2
figure.
"""
from __future__ import annotations

import numpy as np

L = 16                 # window (state) width in bits
TILE = 16              # tile edge
SEQ = TILE * TILE      # 256 weights per trellis sequence


def words_per_tile(k_bits: int) -> int:
    return 8 * k_bits   # 256 * K bits / 32


def stream_bits(words: np.ndarray, k_bits: int) -> np.ndarray:
    """Unpack tiles of 8K words into bit strings. words: uint32 [..., 8K] -> uint8 [..., 256K]."""
    w = np.asarray(words, dtype=np.uint32)
    assert w.shape[-1] == words_per_tile(k_bits)
    # big-endian byte order puts each word's bit 31 first; unpackbits reads each byte MSB first
    be = np.ascontiguousarray(w.astype(">u4")).view(np.uint8)
    return np.unpackbits(be, axis=-1)


def step(state: np.ndarray, new_bits: np.ndarray, b: int, width: int = L) -> np.ndarray:
    """One trellis transition ([DD] Section 3): shift left by b, keep `width` bits, OR in b new bits."""
    s = np.asarray(state, dtype=np.int64)
    return ((s << b) & ((1 << width) - 1)) | np.asarray(new_bits, dtype=np.int64)


def _bits_to_int(bits: np.ndarray) -> np.ndarray:
    """Most-significant-first bit vector(s) along the last axis -> integer."""
    out = np.zeros(bits.shape[:-1], dtype=np.int64)
    for j in range(bits.shape[-1]):
        out = (out << 1) | bits[..., j].astype(np.int64)
    return out


def walk_states(bits: np.ndarray, k_bits: int, v: int = 1) -> np.ndarray:
    """Walk the tail-biting trellis state by state. bits uint8 [..., 256K] -> states int64 [..., 256/v].

    S_0 is the first 16 bits of the circle; each later state shifts in the
    next b = v*K bits, taken cyclically.
    """
    nbits = bits.shape[-1]
    assert nbits == SEQ * k_bits
    b, nsteps = v * k_bits, SEQ // v
    states = np.empty(bits.shape[:-1] + (nsteps,), dtype=np.int64)
    s = _bits_to_int(bits[..., :L])
    states[..., 0] = s
    for t in range(1, nsteps):
        first = L + b * (t - 1)                                   # next unread bit of the circle
        idx = [(first + i) % nbits for i in range(b)]
        s = step(s, _bits_to_int(bits[..., idx]), b)
        states[..., t] = s
    return states


def window_states(bits: np.ndarray, k_bits: int, v: int = 1) -> np.ndarray:
    """Random-access route ([TQ] Part eight): S_t = 16-bit window starting at bit v*K*t of the circle."""
    nbits = bits.shape[-1]
    t = np.arange(SEQ // v)
    idx = (v * k_bits * t[:, None] + np.arange(L)[None, :]) % nbits   # [256/v, 16]
    return _bits_to_int(bits[..., idx])


def stream_from_states(states: np.ndarray, k_bits: int, v: int = 1) -> np.ndarray:
    """Inverse map: concatenating the top v*K bits of every state gives back the 256K-bit stream."""
    s = np.asarray(states, dtype=np.int64)
    b = v * k_bits
    cols = [((s >> (L - 1 - i)) & 1) for i in range(b)]            # [..., 256/v] each
    return np.stack(cols, axis=-1).reshape(*s.shape[:-1], SEQ * k_bits).astype(np.uint8)


def is_valid_path(states: np.ndarray, k_bits: int, v: int = 1) -> np.ndarray:
    """True where every consecutive pair (cyclically) is a bitshift-trellis edge.

    S_{t+1} must keep the low 16-b bits of S_t as its top 16-b bits (b = v*K).
    """
    s = np.asarray(states, dtype=np.int64)
    b = v * k_bits
    nxt = np.roll(s, -1, axis=-1)
    keep = (1 << (L - b)) - 1
    return np.all((nxt >> b) == (s & keep), axis=-1)


def closes_circle(states: np.ndarray, bits: np.ndarray, k_bits: int, v: int = 1) -> np.ndarray:
    """Tail-biting closure: stepping the last state with bits 16-b..15 of the circle gives S_0 again."""
    b = v * k_bits
    tail = _bits_to_int(bits[..., L - b:L])
    return step(states[..., -1], tail, b) == states[..., 0]


def tile_index(R: int, C: int, n: int) -> int:
    return R * (n // TILE) + C


def layer_states(codes: np.ndarray, m: int, n: int, k_bits: int, tile_rows=None, v: int = 1) -> np.ndarray:
    """States of a whole layer (or of the listed tile rows) by walking every tile.

    Returns int64 [len(tile_rows), n/16, 256/v] with tile_rows defaulting to all m/16.
    """
    wpt = words_per_tile(k_bits)
    tiles = np.asarray(codes, dtype=np.uint32).reshape(m // TILE, n // TILE, wpt)
    if tile_rows is not None:
        tiles = tiles[np.asarray(tile_rows)]
    return walk_states(stream_bits(tiles, k_bits), k_bits, v)


def states_to_matrix(states: np.ndarray) -> np.ndarray:
    """[R, C, 256] per-tile sequences (t = 16r + c) -> [16R, 16C] row-major matrix."""
    R, C, _ = states.shape
    return states.reshape(R, C, TILE, TILE).transpose(0, 2, 1, 3).reshape(R * TILE, C * TILE)

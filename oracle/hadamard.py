"""Randomized Hadamard transform on 128-blocks (test infrastructure).

Follows [DD] Section 2: the weight matrix is rotated on both sides by a
normalised Walsh-Hadamard matrix (H H^T = I) times a diagonal of random +-1
signs stored as one bit per row / column, and the rotation is undone on the
activations at run time. [TQ] Part eleven: EXL3 rotates blocks of 128 along
each axis rather than whole rows and columns.

Readings where the pages leave it open: Sylvester (natural) ordering,
H[i, j] = (-1)^popcount(i AND j) / sqrt(128); sign bit i is bit i mod 32 of
word i // 32, set meaning -1. The two runtime equations of [DD] Section 2 are
not inverse to each other as printed; the oracle uses
    x~ = blockdiag(H) diag(s_in) x            (input side, as the runtime equation)
    y  = diag(s_out) blockdiag(H) y~          (exact inverse of the left factor H_m diag(s_left))
with H symmetric, so H^T = H.

The matrix is built explicitly and applied as a dense 128x128 product per
block -- no fast transform. Pins (tests/test_oracle_hadamard.py): H H^T = 128 I
for the +-1 form, symmetry, first row constant, agreement with an
independently coded recursive Sylvester construction, forward o inverse =
identity, and the all-ones vector mapping to sqrt(128) e_0.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


def hadamard(n: int = BLOCK) -> np.ndarray:
    """Normalised Sylvester-Hadamard matrix of order n (a power of two), float64."""
    i = np.arange(n)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0) / np.sqrt(n)


def signs(words: np.ndarray, count: int) -> np.ndarray:
    """+-1 float64 vector of length `count` from packed sign words (bit set -> -1)."""
    w = np.asarray(words, dtype=np.uint32)
    i = np.arange(count)
    bit = (w[i // 32] >> (i % 32).astype(np.uint32)) & 1
    return np.where(bit == 1, -1.0, 1.0)


def _blocks(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    assert v.shape[-1] % BLOCK == 0, "length must be a multiple of 128"
    return v.reshape(*v.shape[:-1], v.shape[-1] // BLOCK, BLOCK)


def apply_blocks(v: np.ndarray) -> np.ndarray:
    """blockdiag(H, ..., H) @ v along the last axis (dense product per block)."""
    H = hadamard(BLOCK)
    b = _blocks(v)
    return (b @ H.T).reshape(np.shape(v))


def hadamard_pm1(n: int = BLOCK) -> np.ndarray:
    """Unnormalised Sylvester-Hadamard matrix of order n: entries exactly +1 / -1 (float64)."""
    i = np.arange(n)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def apply_blocks_pm1(v: np.ndarray) -> np.ndarray:
    """blockdiag(sqrt(128) H) @ v along the last axis: the +-1 transform without its 1/sqrt(128).

    For binary16 inputs every partial sum is a multiple of 2^-24 below 2^23 in
    magnitude (47 significant bits), so each result is exact in float64 in any
    summation order.
    """
    b = _blocks(v)
    return (b @ hadamard_pm1(BLOCK).T).reshape(np.shape(v))


def rht_forward(x: np.ndarray, sign_words: np.ndarray) -> np.ndarray:
    """Input side: x~ = blockdiag(H) diag(s) x (last axis)."""
    x = np.asarray(x, dtype=np.float64)
    return apply_blocks(signs(sign_words, x.shape[-1]) * x)


def rht_inverse(v: np.ndarray, sign_words: np.ndarray) -> np.ndarray:
    """Output side: y = diag(s) blockdiag(H) v (last axis)."""
    v = np.asarray(v, dtype=np.float64)
    return signs(sign_words, v.shape[-1]) * apply_blocks(v)


def blockdiag_matrix(n: int) -> np.ndarray:
    """Dense blockdiag(H, ..., H) of order n (for the dense route of the GEMV)."""
    H = hadamard(BLOCK)
    out = np.zeros((n, n))
    for b in range(n // BLOCK):
        out[b * BLOCK:(b + 1) * BLOCK, b * BLOCK:(b + 1) * BLOCK] = H
    return out

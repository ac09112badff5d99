"""The computed code: 16-bit trellis state -> fp16 weight (test infrastructure).

Follows the three-instruction code of [TQ] Part nine (and its self-check
answer seven): (1) one step of a 32-bit linear congruential generator, a
single multiply-add of the state; (2) treat the 32 bits as two 16-bit halves,
keep each half's sign bit and low bits with a mask and XOR in a constant that
pins the exponent, giving two half-precision values with random signs and
bounded magnitude; (3) add the two halves with one half-precision add.
Step (2) is the mantissa-splice trick of [TQ] Part three.

The pages print no constants for this code. Reading where they leave it open:
the multiplier is the blog's 0x9E3779B9 ([DD] Section 3 code) cut to its top
24 bits, 0x9E3779, so the multiply-add is one full-rate instruction on the
target, as [TQ] Part nine requires of step (1); the addend is the blog's
0x7F4A7C15; the mask 0x8FFF8FFF keeps each half's sign, the two low exponent
bits and the 10 fraction bits; the XOR constant 0x30003000 forces exponent
field 0b011xx, so each half lies in +-[1/8, 2). The sum is rounded to
binary16 with ties to even.

Pins (tests/test_oracle_code.py): hand-derived values for chosen states
(tests/golden/code_hand_values.txt); NumPy's independent float16 rounding on
all 65,536 states; structural invariants the pages state (bounded halves,
random balanced signs, near-Gaussian sum); no NaN / infinity / subnormal.
"""
from __future__ import annotations

import numpy as np

from . import fp16

MUL = 0x009E3779          # LCG multiplier (24 bits)
ADD = 0x7F4A7C15          # LCG addend
MASK = 0x8FFF8FFF         # keep sign + low 2 exponent bits + 10 fraction bits of each half
XOR = 0x30003000          # pins each half's exponent field to 0b011xx

_M32 = (1 << 32) - 1


def lcg(states) -> np.ndarray:
    """Step (1): h = (MUL * S + ADD) mod 2^32, exact in int64 (product < 2^40)."""
    s = np.asarray(states, dtype=np.int64)
    return (s * MUL + ADD) & _M32


def mask_xor(h) -> np.ndarray:
    """Step (2): u = (h AND MASK) XOR XOR."""
    return (np.asarray(h, dtype=np.int64) & MASK) ^ XOR


def halves(u):
    """Low and high 16-bit halves of u as binary16 bit patterns."""
    u = np.asarray(u, dtype=np.int64)
    return (u & 0xFFFF).astype(np.uint16), ((u >> 16) & 0xFFFF).astype(np.uint16)


def weight_bits(states) -> np.ndarray:
    """Step (3): fp16 bits of RNE(value(lo) + value(hi)).

    The exact sum is formed in float64 (both halves are multiples of 2^-13
    below 2 in magnitude, so the float64 sum is exact) and then rounded once.
    """
    lo, hi = halves(mask_xor(lcg(states)))
    return fp16.round_rne(fp16.value(lo) + fp16.value(hi))


def weight_values(states) -> np.ndarray:
    """Decoded weights as exact float64 values."""
    return fp16.value(weight_bits(states))


def table() -> np.ndarray:
    """The whole code: fp16 bits for all 65,536 states."""
    return weight_bits(np.arange(1 << 16))


# ---------------------------------------------------------------------------
# code_id 1, the pair code (this library's V=2 variant of the pages' vector trellis, a reading):
# one state per two consecutive weights ([DD] Section 3: b*V bits per
# V-dimensional step; its decode snippet yields a pair of halves per state).
# The state goes through the same multiply-add and mask/XOR; the halves a, b
# give the rotated pair (a + b, b - a), each rounded to binary16 -- every
# weight is again a sum of two bounded halves ([TQ] Part nine).
# Pins (tests/test_oracle_code.py): hand-derived values
# (tests/golden/pair_code_hand_values.txt), NumPy's float16 cast on all states,
# the pair's sum/difference identities.
# ---------------------------------------------------------------------------

def pair_weight_bits(states):
    """fp16 bits of (RNE(a + b), RNE(b - a)) for each state; returns two arrays."""
    lo, hi = halves(mask_xor(lcg(states)))
    a, b = fp16.value(lo), fp16.value(hi)
    return fp16.round_rne(a + b), fp16.round_rne(b - a)


def pair_table() -> np.ndarray:
    """The pair code for all states: uint16 [65536, 2] = (even weight, odd weight)."""
    e, o = pair_weight_bits(np.arange(1 << 16))
    return np.stack([e, o], axis=-1)


# ---------------------------------------------------------------------------
# code_id 2, "mul1": the EXL3 converter's default codebook ([FG] "What the EXL3
# converter actually sets"; [TQ] Part eleven, Part twelve). Steps, as the pages
# describe them: (1) multiply the state by a constant with no additive term
# (EXL3's MCG change to the generator); (2) keep the low six bits of each of
# the product's four bytes; (3) add the four bytes (one four-byte dot product
# against ones on a GPU) and subtract a fixed offset, giving an integer level
# in [-126, 126] with a bell-shaped spread; the weight is an affine function of
# that level.
# Readings where the pages leave it open: the multiplier is code 0's 0x9E3779
# (the pages print no constant for mul1 either); the offset is 126, the mean
# of four uniform six-bit bytes, so the levels are symmetric; the weight is the
# level times 1/32, exact in binary16 (|w| <= 126/32), so no rounding is
# involved anywhere.
# Pins (tests/test_oracle_code.py): hand-worked values
# (tests/golden/mul1_hand_values.txt); all 65,536 states against a separate
# pure-Python integer byte sum; the level histogram against the exact
# distribution of a sum of four independent uniform six-bit bytes.
# ---------------------------------------------------------------------------

BYTE_MASK = 0x3F3F3F3F    # low six bits of each byte
MUL1_OFFSET = 126
MUL1_STEP = 1.0 / 32.0    # weight per level


def mcg(states) -> np.ndarray:
    """Step (1): h = (MUL * S) mod 2^32, the multiply with the additive constant dropped."""
    s = np.asarray(states, dtype=np.int64)
    return (s * MUL) & _M32


def byte_sum(h) -> np.ndarray:
    """Step (2) and the sum of step (3): sum of the four bytes of (h AND 0x3F3F3F3F), in 0..252."""
    m = np.asarray(h, dtype=np.int64) & BYTE_MASK
    return (m & 0xFF) + ((m >> 8) & 0xFF) + ((m >> 16) & 0xFF) + ((m >> 24) & 0xFF)


def mul1_level(states) -> np.ndarray:
    """Integer level of each state: byte sum minus the offset, in -126..126."""
    return byte_sum(mcg(states)) - MUL1_OFFSET


def mul1_bits(states) -> np.ndarray:
    """fp16 bits of the weight level / 32 (exact: a multiple of 2^-5 below 4 in magnitude)."""
    return fp16.round_rne(mul1_level(states).astype(np.float64) * MUL1_STEP)


def mul1_table() -> np.ndarray:
    """code_id 2 for all states: fp16 bits [65536]."""
    return mul1_bits(np.arange(1 << 16))


# ---------------------------------------------------------------------------
# code_id 3, "MCG": EXL3's variant of the three-instruction code ([TQ] Part
# eleven: the generator keeps only the multiply, the additive constant is
# dropped; [FG] "What the EXL3 converter actually sets": one of the converter's
# three codebook names). Steps: (1) h = multiplier * S mod 2^32; (2) and (3) as
# for code 0: mask/XOR each half into a bounded binary16 value and add the two
# halves with one binary16 add.
# Reading where the pages leave it open: the multiplier is code 0's 0x9E3779
# (the pages mention a 32-bit constant without printing it; 24 bits keep the
# multiply one full-rate instruction, as for code 0 and mul1).
# Pins (tests/test_oracle_code.py): hand-worked values
# (tests/golden/mcg_hand_values.txt); NumPy's float16 cast on all states; the
# generator's linearity (no additive constant: h(a + b) = h(a) + h(b) mod 2^32);
# the same bounds and balance as code 0.
# ---------------------------------------------------------------------------

def mcg_weight_bits(states) -> np.ndarray:
    """fp16 bits of RNE(value(lo) + value(hi)) with the halves of (mcg(S) AND MASK) XOR XOR."""
    lo, hi = halves(mask_xor(mcg(states)))
    return fp16.round_rne(fp16.value(lo) + fp16.value(hi))


def mcg_table() -> np.ndarray:
    """code_id 3 for all states: fp16 bits [65536]."""
    return mcg_weight_bits(np.arange(1 << 16))


CODE_V = {0: 1, 1: 2, 2: 1, 3: 1}     # weights per trellis step of each code_id

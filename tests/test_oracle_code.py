"""Pins for the oracle's computed code and its binary16 helpers (no GPU)."""
from fractions import Fraction

import numpy as np

from conftest import golden_rows
from oracle import code, fp16


def test_hand_values():
    """Every intermediate of the three-instruction code against hand-derived values."""
    for state, h, u, lo, hi, num, den, w in golden_rows("code_hand_values.txt"):
        s = np.array([int(state, 16)])
        assert int(code.lcg(s)[0]) == int(h, 16)
        assert int(code.mask_xor(code.lcg(s))[0]) == int(u, 16)
        l, hh = code.halves(code.mask_xor(code.lcg(s)))
        assert int(l[0]) == int(lo, 16) and int(hh[0]) == int(hi, 16)
        total = fp16.value(l) + fp16.value(hh)
        assert Fraction(float(total[0])) == Fraction(int(num), int(den))
        assert int(code.weight_bits(s)[0]) == int(w, 16)


def test_mask_and_xor_are_disjoint():
    """XOR into masked-off bits equals OR: the pages' mask-then-XOR is one bit-insert."""
    assert code.MASK & code.XOR == 0
    assert code.MUL < 1 << 24


def test_table_rounding_matches_numpy_cast():
    """The oracle's own round-to-nearest-even against NumPy's float64->float16 cast, all states."""
    lo, hi = code.halves(code.mask_xor(code.lcg(np.arange(1 << 16))))
    exact = fp16.value(lo) + fp16.value(hi)
    assert (fp16.round_rne(exact) == exact.astype(np.float16).view(np.uint16)).all()
    assert (code.table() == exact.astype(np.float16).view(np.uint16)).all()


def test_fp16_value_matches_numpy_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = fp16.value(bits)
    ref = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    assert (ours[fin] == ref[fin]).all()
    assert (np.isnan(ours) == np.isnan(ref)).all()


def test_round_rne_edge_cases():
    cases = [(0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3C00), (65504.0, 0x7BFF), (65520.0, 0x7C00),
             (65519.99, 0x7BFF), (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (3 * 2.0 ** -25, 0x0002),
             (2.0 ** -14, 0x0400), (1.0 + 2.0 ** -11, 0x3C00), (1.0 + 3 * 2.0 ** -11, 0x3C02),
             (-2.8427734375, 0xC1B0)]
    for v, b in cases:
        assert int(fp16.round_rne(np.array([v]))[0]) == b, v
    rng = np.random.default_rng(0)
    v = rng.standard_normal(100000) * rng.choice([1e-6, 1e-3, 1, 1e3], 100000)
    assert (fp16.round_rne(v) == v.astype(np.float16).view(np.uint16)).all()


def test_halves_are_bounded_signed_and_exponent_pinned():
    """Each half keeps its sign, has exponent field 0b011xx (|half| in [1/8, 2)); no NaN/Inf/subnormal."""
    u = code.mask_xor(code.lcg(np.arange(1 << 16)))
    for half in code.halves(u):
        e = (half.astype(np.int64) >> 10) & 0x1F
        assert set(np.unique(e)) <= {12, 13, 14, 15}
        v = np.abs(fp16.value(half))
        assert v.min() >= 0.125 and v.max() < 2.0
    lo, hi = code.halves(u)
    # the multiplier is odd, so S -> low 16 bits of h is a bijection: the low half's sign is exactly balanced
    assert ((lo >> 15) == 1).sum() == 1 << 15
    assert abs(((hi >> 15) == 1).mean() - 0.5) < 0.01


def test_sum_is_near_gaussian_and_finite():
    """The sum of the two halves is close to a Gaussian (lecture, Part nine)."""
    w = fp16.value(code.table())
    assert np.isfinite(w).all()
    e = (code.table().astype(np.int64) >> 10) & 0x1F
    assert not ((e == 0) & ((code.table() & 0x3FF) != 0)).any()    # no subnormals
    assert abs(w.mean()) < 0.01
    assert 1.1 < w.std() < 1.4
    kurt = ((w - w.mean()) ** 4).mean() / w.var() ** 2
    assert 2.5 < kurt < 3.5
    assert np.abs(w).max() < 4.0


def test_pair_code_hand_values():
    """The pair code (code_id 1): rotated pair of the two halves, each rounded to binary16."""
    for state, lo, hi, en, ed, we, on, od, wo in golden_rows("pair_code_hand_values.txt"):
        s = np.array([int(state, 16)])
        l, h = code.halves(code.mask_xor(code.lcg(s)))
        assert int(l[0]) == int(lo, 16) and int(h[0]) == int(hi, 16)
        e, o = code.pair_weight_bits(s)
        assert int(e[0]) == int(we, 16) and int(o[0]) == int(wo, 16)
        a, b = fp16.value(l)[0], fp16.value(h)[0]
        assert Fraction(float(a + b)) == Fraction(int(en), int(ed))
        assert Fraction(float(b - a)) == Fraction(int(on), int(od))


def test_pair_table_matches_numpy_and_is_balanced():
    lo, hi = code.halves(code.mask_xor(code.lcg(np.arange(1 << 16))))
    a = lo.view(np.float16).astype(np.float64)
    b = hi.view(np.float16).astype(np.float64)
    t = code.pair_table()
    assert (t[:, 0] == (a + b).astype(np.float16).view(np.uint16)).all()
    assert (t[:, 1] == (b - a).astype(np.float16).view(np.uint16)).all()
    # the even weight is the V=1 code's weight for the same state
    assert (t[:, 0] == code.table()).all()
    we, wo = fp16.value(t[:, 0]), fp16.value(t[:, 1])
    for w in (we, wo):
        assert np.isfinite(w).all() and abs(w.mean()) < 0.02 and 1.1 < w.std() < 1.4
    assert abs(np.corrcoef(we, wo)[0, 1]) < 0.05


# --- code_id 2, mul1 ----------------------------------------------------------------------

def test_mul1_hand_values():
    """Every intermediate of mul1 against the hand-worked fixture."""
    for state, h, m, b0, b1, b2, b3, sig, lev, w in golden_rows("mul1_hand_values.txt"):
        s = np.array([int(state, 16)])
        assert int(code.mcg(s)[0]) == int(h, 16)
        assert int(code.mcg(s)[0]) & code.BYTE_MASK == int(m, 16)
        assert sum(int(v) for v in (b0, b1, b2, b3)) == int(sig)
        assert int(code.byte_sum(code.mcg(s))[0]) == int(sig)
        assert int(code.mul1_level(s)[0]) == int(lev)
        assert int(code.mul1_bits(s)[0]) == int(w, 16)


def test_mul1_all_states_against_python_byte_sum():
    """All 65,536 states against a separate route: Python integers, bytes() and a per-byte mask."""
    ref = []
    for s in range(1 << 16):
        h = (0x9E3779 * s) % (1 << 32)
        ref.append(sum(b & 0x3F for b in h.to_bytes(4, "little")) - 126)
    ref = np.array(ref)
    assert (code.mul1_level(np.arange(1 << 16)) == ref).all()
    exact = ref / 32.0
    assert (code.mul1_table() == exact.astype(np.float16).view(np.uint16)).all()
    assert (fp16.value(code.mul1_table()) == exact).all()       # no rounding anywhere


def test_mul1_levels_follow_four_uniform_bytes():
    """The level histogram over all states against the exact law of a sum of four independent
    uniform six-bit bytes (the bell shape the pages describe), and its symmetry."""
    law = np.ones(64)
    for _ in range(3):
        law = np.convolve(law, np.ones(64))
    law /= law.sum()                                   # P(sigma = s), s = 0..252
    lev = code.mul1_level(np.arange(1 << 16))
    assert lev.min() >= -126 and lev.max() <= 126
    hist = np.bincount(lev + 126, minlength=253) / lev.size
    assert 0.5 * np.abs(hist - law).sum() < 0.03      # total variation distance
    assert abs(lev.mean()) < 0.5 and abs(lev.std() - np.sqrt(4 * (64 ** 2 - 1) / 12)) < 1.0
    assert code.mul1_level(np.array([0]))[0] == -126   # multiply-only: state 0 stays 0


# --- code_id 3, MCG ------------------------------------------------------------------------

def test_mcg_hand_values():
    """Every intermediate of MCG against the hand-worked fixture (a tie, the fixed point, a zero sum)."""
    for state, h, u, lo, hi, num, den, w in golden_rows("mcg_hand_values.txt"):
        s = np.array([int(state, 16)])
        assert int(code.mcg(s)[0]) == int(h, 16)
        assert int(code.mask_xor(code.mcg(s))[0]) == int(u, 16)
        l, hh = code.halves(code.mask_xor(code.mcg(s)))
        assert int(l[0]) == int(lo, 16) and int(hh[0]) == int(hi, 16)
        total = fp16.value(l) + fp16.value(hh)
        assert Fraction(float(total[0])) == Fraction(int(num), int(den))
        assert int(code.mcg_weight_bits(s)[0]) == int(w, 16)


def test_mcg_all_states_against_python_integers_and_numpy_cast():
    """All 65,536 states by a separate route: Python integers for the hash and the bit logic,
    NumPy's float16 view and cast for the halves and the rounding."""
    lo = np.empty(1 << 16, np.uint16)
    hi = np.empty(1 << 16, np.uint16)
    for s in range(1 << 16):
        u = (((0x9E3779 * s) % (1 << 32)) & 0x8FFF8FFF) | 0x30003000   # disjoint mask/XOR: OR
        lo[s], hi[s] = u & 0xFFFF, u >> 16
    exact = lo.view(np.float16).astype(np.float64) + hi.view(np.float16).astype(np.float64)
    assert (code.mcg_table() == exact.astype(np.float16).view(np.uint16)).all()


def test_mcg_generator_is_linear():
    """No additive constant: h(a + b) = h(a) + h(b) and h(2a) = 2 h(a) mod 2^32, h(0) = 0
    (each fails for the three-instruction code's multiply-add)."""
    rng = np.random.default_rng(5)
    a = rng.integers(0, 1 << 15, 4096)
    b = rng.integers(0, 1 << 15, 4096)
    m32 = (1 << 32) - 1
    assert ((code.mcg(a) + code.mcg(b)) & m32 == code.mcg(a + b)).all()
    assert ((2 * code.mcg(a)) & m32 == code.mcg(2 * a)).all()
    assert code.mcg(np.array([0]))[0] == 0
    assert not ((code.lcg(a) + code.lcg(b)) & m32 == code.lcg(a + b)).any()


def test_mcg_halves_bounded_balanced_and_sum_near_gaussian():
    """Same structure as code 0: halves in +-[1/8, 2), the low half's sign exactly balanced
    (odd multiplier: S -> h mod 2^16 is a bijection), a finite near-Gaussian sum."""
    u = code.mask_xor(code.mcg(np.arange(1 << 16)))
    lo, hi = code.halves(u)
    for half in (lo, hi):
        v = np.abs(fp16.value(half))
        assert v.min() >= 0.125 and v.max() < 2.0
    assert ((lo >> 15) == 1).sum() == 1 << 15
    assert abs(((hi >> 15) == 1).mean() - 0.5) < 0.01
    w = fp16.value(code.mcg_table())
    assert np.isfinite(w).all() and abs(w.mean()) < 0.01 and 1.1 < w.std() < 1.4
    kurt = ((w - w.mean()) ** 4).mean() / w.var() ** 2
    assert 2.5 < kurt < 3.5
    # it is a different code from code 0 on almost every state
    assert (code.mcg_table() != code.table()).mean() > 0.99

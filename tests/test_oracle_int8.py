"""Pins for the oracle's int8-activation form of the product (no GPU).

The quantiser (oracle.gemv.quantize_rotated) is checked against a separate route
written here with exact fractions, explicit +-1 Hadamard signs from popcounts
and Python's round() (which rounds halves to even); the product against the
plain GEMV in cases where quantising loses nothing, and against the half-step
error bound otherwise.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import fp16, gemv, hadamard
from trellis_coded_gemv_amd import inputs


def _layer(n, seed, m=128):
    return inputs.make_layer(m, n, 2, seed, code_id=2)


def _route_by_fractions(x_bits, sign_words, n):
    """u, e, q for one vector, with Fractions and loops only."""
    xv = [Fraction(float(v)) for v in np.asarray(x_bits, np.uint16).view(np.float16)]
    sgn = [-1 if (int(sign_words[i // 32]) >> (i % 32)) & 1 else 1 for i in range(n)]
    u, es, qs = [], [], []
    for b in range(n // 128):
        ub = []
        for i in range(128):
            tot = Fraction(0)
            for j in range(128):
                h = -1 if bin(i & j).count("1") % 2 else 1
                tot += h * sgn[128 * b + j] * xv[128 * b + j]
            ub.append(tot)
        amax = max(abs(v) for v in ub)
        e = 0
        if amax:
            e = -60
            while amax / Fraction(2) ** e > 127:
                e += 1
        u += ub
        es.append(e)
        qs += [round(v / Fraction(2) ** e) for v in ub]
    return u, es, qs


def test_pm1_transform_is_exact_over_wide_exponent_range():
    rng = np.random.default_rng(11)
    mag = np.exp2(rng.integers(-24, 15, 128).astype(np.float64)) * rng.choice([-1, 1], 128)
    x = (mag * rng.uniform(1, 2, 128)).astype(np.float16)
    xv = [Fraction(float(v)) for v in x]
    u = hadamard.apply_blocks_pm1(x.astype(np.float64))
    for i in (0, 1, 77, 127):
        ref = sum((-1 if bin(i & j).count("1") % 2 else 1) * xv[j] for j in range(128))
        assert Fraction(float(u[i])) == ref


@pytest.mark.parametrize("seed", [0, 1])
def test_quantizer_against_fraction_route(seed):
    n = 256
    layer = _layer(n, 300 + seed)
    x = inputs.make_x(n, 310 + seed)
    q, e = gemv.quantize_rotated(layer, x)
    _, es, qs = _route_by_fractions(x, layer.sign_in, n)
    assert list(e) == es
    assert list(q) == qs


def test_ties_round_to_even():
    """u = a +- b on alternate rows of the first block: exact halves after scaling by 2^0."""
    n = 256
    layer = _layer(n, 320)
    layer.sign_in[:] = 0                           # all signs +1
    x = np.zeros(n, np.float16)
    x[0], x[1] = 100.5, 25.0                       # block 0: u = 125.5 (even rows), 75.5 (odd rows)
    x[128], x[129] = 100.5, 26.0                   # block 1: u = 126.5, 74.5
    q, e = gemv.quantize_rotated(layer, x.view(np.uint16))
    assert list(e) == [0, 0]
    assert set(q[0:128:2]) == {126} and set(q[1:128:2]) == {76}
    assert set(q[128::2]) == {126} and set(q[129::2]) == {74}
    _, _, qs = _route_by_fractions(x.view(np.uint16), layer.sign_in, n)
    assert list(q) == qs


def test_lossless_when_integer_and_small():
    """Integer u with max |u| <= 127 quantises exactly (e <= 0): the int8 product is the GEMV."""
    n = 384
    layer = _layer(n, 330, m=256)
    rng = np.random.default_rng(5)
    x = np.zeros(n, np.float16)
    idx = rng.choice(n, 40, replace=False)
    x[idx] = rng.integers(-2, 3, 40)
    q, e = gemv.quantize_rotated(layer, x.view(np.uint16))
    assert (e <= 0).all()
    y = gemv.gemv(layer, x.view(np.uint16))
    yi = gemv.gemv_int8(layer, x.view(np.uint16))
    assert np.abs(yi - y).max() <= 1e-12 * np.abs(y).max()


def test_half_step_bound_and_tight_scale():
    n = 1024
    layer = _layer(n, 340)
    x = inputs.make_x(n, 341)
    q, e = gemv.quantize_rotated(layer, x)
    xt = hadamard.rht_forward(fp16.value(x), layer.sign_in)
    xh = gemv.dequantized(q, e)
    step = np.repeat(np.exp2(e.astype(np.float64)), 128) / np.sqrt(128)
    assert (np.abs(xh - xt) <= 0.5 * step * (1 + 1e-12)).all()
    qa = np.abs(q).reshape(-1, 128).max(axis=1)
    assert ((qa >= 64) & (qa <= 127)).all()


def test_zero_block_and_rows_route():
    n = 256
    layer = _layer(n, 350, m=256)
    x = inputs.make_x(n, 351).copy()
    x[128:] = 0
    q, e = gemv.quantize_rotated(layer, x)
    assert e[1] == 0 and (q[128:] == 0).all()
    rows = np.arange(256)
    assert np.abs(gemv.gemv_int8_rows(layer, x, rows) - gemv.gemv_int8(layer, x)).max() < 1e-12

"""Pins for the oracle's mixture-of-experts block (no GPU)."""
import numpy as np

from oracle import fp16, gemv, moe
from trellis_coded_gemv_amd import inputs


def test_silu_closed_forms():
    assert moe.silu(0.0) == 0.0
    assert abs(moe.silu(40.0) - 40.0) < 1e-12 and abs(moe.silu(-40.0)) < 1e-15
    v = np.linspace(-6, 6, 25)
    assert np.allclose(moe.silu(v) - moe.silu(-v), v)              # silu(v) - silu(-v) = v
    assert np.isclose(moe.silu(1.0), 1.0 / (1.0 + np.exp(-1.0)))
    assert np.isclose(moe.silu(np.log(3.0)), np.log(3.0) * 0.75)   # sigmoid(ln 3) = 3/4


def _experts(n, hidden=256, inter=128, seed=60):
    gu = [inputs.make_layer(inter, hidden, 1 + (i % 3), seed, tensor=i) for i in range(2 * n)]
    dn = [inputs.make_layer(hidden, inter, 1 + (i % 2), seed, tensor=100 + i) for i in range(n)]
    return gu, dn


def test_single_expert_is_the_chain_of_gemvs():
    gu, dn = _experts(3)
    x = inputs.make_x(256, 61)
    g = gemv.gemv(gu[2], x)
    u = gemv.gemv(gu[3], x)
    h = fp16.round_rne(g / (1 + np.exp(-g)) * u)
    y = moe.moe_block(gu, dn, [1], [1.0], x)
    assert np.array_equal(y, gemv.gemv(dn[1], h))


def test_linear_in_router_weights_and_order_free():
    gu, dn = _experts(4)
    x = inputs.make_x(256, 62)
    y1 = moe.moe_block(gu, dn, [3], [1.0], x)
    y2 = moe.moe_block(gu, dn, [0], [1.0], x)
    y = moe.moe_block(gu, dn, [3, 0], [0.25, 0.75], x)
    assert np.allclose(y, 0.25 * y1 + 0.75 * y2, rtol=1e-12, atol=1e-12)
    yr = moe.moe_block(gu, dn, [0, 3], [0.75, 0.25], x)
    assert np.allclose(y, yr, rtol=1e-12, atol=1e-12)
    assert np.array_equal(moe.moe_block(gu, dn, [2], [0.0], x), np.zeros(256))

"""Pins for the oracle's mixture-of-experts block (no GPU)."""
import numpy as np

from conftest import hand_code
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


def _zero_stream_expert_set(n_experts, hidden=256, inter=256, seed=64):
    """Experts whose every stream is all zeros (every state 0), with one scale per tensor on
    every output: 2^-10 for gate and down, 1.5 * 2^-10 for up (so gate and up differ)."""
    def zl(m, n, t, g):
        L = inputs.make_layer(m, n, 2, seed, tensor=t)
        L.codes = np.zeros(inputs.words_per_layer(m, n, 2), np.uint32)
        L.scales = np.full(m, np.float16(g).view(np.uint16), np.uint16)
        return L
    gu = [zl(inter, hidden, i, 2.0 ** -10 * (1.5 if i % 2 else 1.0)) for i in range(2 * n_experts)]
    dn = [zl(hidden, inter, 100 + i, 2.0 ** -10) for i in range(n_experts)]
    return gu, dn


def _signs(words, n):
    i = np.arange(n)
    return 1.0 - 2.0 * ((words[i // 32] >> (i % 32)) & 1).astype(np.float64)


def _zero_stream_gemv(L, xv):
    """Closed form of a zero-stream GEMV (all weights w0 = code(0), constant scale g):
    y_o = s_out[o] g w0 128 sum_b s_in[128 b] x[128 b] for o = 0 mod 128, else 0."""
    w0 = hand_code(0)
    g = float(L.scales[:1].view(np.float16)[0])
    s_in, s_out = _signs(L.sign_in, L.n), _signs(L.sign_out, L.m)
    sigma = sum(s_in[128 * b] * xv[128 * b] for b in range(L.n // 128))
    y = np.zeros(L.m)
    y[::128] = s_out[::128] * g * w0 * 128.0 * sigma
    return y


def test_zero_stream_block_closed_form():
    """Whole block on zero streams, by hand: gate and up are non-zero only at o = 0 mod 128,
    so is h = fp16(silu(gate) * up) (silu from scipy's logistic, fp16 by NumPy's cast), and
    the down projection's closed form gives y. Fails if gate and up are swapped, if silu acts
    on up, or if h is not rounded to binary16 once."""
    from scipy.special import expit
    gu, dn = _zero_stream_expert_set(3)
    x = inputs.make_x(256, 65)
    xv = x.view(np.float16).astype(np.float64)
    sel, wts = [2, 0], [0.3, 0.7]
    expect = np.zeros(256)
    for e, w in zip(sel, wts):
        G = _zero_stream_gemv(gu[2 * e], xv)
        U = _zero_stream_gemv(gu[2 * e + 1], xv)
        assert np.count_nonzero(G) == 2 and not np.allclose(np.abs(G), np.abs(U))
        h = (G * expit(G) * U).astype(np.float16).astype(np.float64)
        assert np.count_nonzero(h) == 2
        expect += w * _zero_stream_gemv(dn[e], h)
    y = moe.moe_block(gu, dn, sel, wts, x)
    assert np.abs(expect).max() > 0
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-12 * np.abs(expect).max())

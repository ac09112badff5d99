"""Pins for the oracle's full matrix-vector product (no GPU)."""
import numpy as np
import pytest

from conftest import golden_rows
from oracle import fp16, gemv
from trellis_coded_gemv_amd import inputs

SQ = np.sqrt(128.0)


def _hand_code(state):
    """Weight value for a state, from the hand-derived golden fixture (not the oracle)."""
    for row in golden_rows("code_hand_values.txt"):
        if int(row[0], 16) == state:
            return float(np.array([int(row[7], 16)], np.uint16).view(np.float16)[0])
    raise KeyError(state)


def _sylvester_pm(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def _layer(m, n, k, codes=None, scales=None, sign_in=None, sign_out=None, seed=7):
    L = inputs.make_layer(m, n, k, seed)
    if codes is not None:
        L.codes = codes
    if scales is not None:
        L.scales = scales
    if sign_in is not None:
        L.sign_in = sign_in
    if sign_out is not None:
        L.sign_out = sign_out
    return L


def _bits(v):
    return np.asarray(v, dtype=np.float16).view(np.uint16)


def test_all_zero_stream_closed_form():
    """All-zero stream: every state is 0, W^ = w0 * 1 1^T, and with g = 1

        y_o = s_out[o] * w0 * sqrt(128) * sigma  for o = 0 mod 128, else 0,
        sigma = sqrt(128) * sum_b s_in[128 b] * x[128 b].
    """
    m, n, k = 256, 384, 2
    L = _layer(m, n, k, codes=np.zeros(inputs.words_per_layer(m, n, k), np.uint32),
               scales=_bits(np.ones(m)))
    x = inputs.make_x(n, 3)
    w0 = _hand_code(0)
    s_in = 1 - 2 * ((L.sign_in[np.arange(n) // 32] >> (np.arange(n) % 32)) & 1).astype(np.float64)
    s_out = 1 - 2 * ((L.sign_out[np.arange(m) // 32] >> (np.arange(m) % 32)) & 1).astype(np.float64)
    xv = x.view(np.float16).astype(np.float64)
    sigma = SQ * sum(s_in[128 * b] * xv[128 * b] for b in range(n // 128))
    expect = np.zeros(m)
    expect[::128] = s_out[::128] * w0 * SQ * sigma
    y = gemv.gemv(L, x)
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-12 * np.abs(expect).max())


def test_scale_acts_before_output_transform():
    """All-zero stream with random g: the output block is s_out * H(g * c) with c = w0 * sigma.

    Its first entry is c * sum(g_blk) / sqrt(128) and its energy is c^2 * sum(g_blk^2)
    (Parseval) -- both fail if g were applied after the output transform.
    """
    m, n, k = 128, 128, 1
    L = _layer(m, n, k, codes=np.zeros(inputs.words_per_layer(m, n, k), np.uint32))
    x = inputs.make_x(n, 4)
    g = L.scales.view(np.float16).astype(np.float64)
    s_in0 = 1 - 2 * float(L.sign_in[0] & 1)
    s_out0 = 1 - 2 * float(L.sign_out[0] & 1)
    c = _hand_code(0) * SQ * s_in0 * x.view(np.float16).astype(np.float64)[0]
    y = gemv.gemv(L, x)
    assert np.isclose(y[0] * s_out0, c * g.sum() / SQ, rtol=1e-12)
    assert np.isclose((y ** 2).sum(), c * c * (g ** 2).sum(), rtol=1e-12)


def test_one_coded_tile_impulse_response():
    """Zero stream except tile (R, C) all ones: W^ is w0 everywhere but w1 = code(0xFFFF) on that
    tile. With g = 1, no signs and x = e_j, the output follows from the +-1 Sylvester matrix alone."""
    m, n, k = 256, 384, 3
    R, C = 5, 17
    codes = np.zeros(inputs.words_per_layer(m, n, k), np.uint32)
    T = R * (n // 16) + C
    codes[T * 8 * k:(T + 1) * 8 * k] = 0xFFFFFFFF
    L = _layer(m, n, k, codes=codes, scales=_bits(np.ones(m)),
               sign_in=np.zeros(n // 32, np.uint32), sign_out=np.zeros(m // 32, np.uint32))
    w0, w1 = _hand_code(0), _hand_code(0xFFFF)
    Wb = gemv.decode_layer(L)
    expect_w = np.full((m, n), _bits([w0])[0])
    expect_w[16 * R:16 * R + 16, 16 * C:16 * C + 16] = _bits([w1])[0]
    assert np.array_equal(Wb, expect_w)

    P = _sylvester_pm(128)
    for j in (256, 256 + 19, 272 + 3, 5):
        x = np.zeros(n, np.float16)
        x[j] = 1.0
        jb, jj = divmod(j, 128)
        xt = np.zeros(n)
        xt[128 * jb:128 * jb + 128] = P[:, jj] / SQ              # H e_j
        yt = np.full(m, w0 * xt.sum())
        yt[16 * R:16 * R + 16] += (w1 - w0) * xt[16 * C:16 * C + 16].sum()
        expect = np.concatenate([P @ yt[b:b + 128] / SQ for b in range(0, m, 128)])
        y = gemv.gemv(L, x.view(np.uint16))
        assert np.allclose(y, expect, atol=1e-12), j


@pytest.mark.parametrize("m,n,k", [(256, 384, 3), (128, 256, 1), (384, 128, 8)])
def test_dense_route_equals_factored_route(m, n, k):
    L = inputs.make_layer(m, n, k, 11)
    x = inputs.make_x(n, 11)
    y = gemv.gemv(L, x)
    yd = gemv.gemv_dense(L, x)
    assert np.abs(y - yd).max() <= 1e-12 * np.abs(y).max()


def test_output_energy_parseval():
    L = inputs.make_layer(256, 256, 2, 12)
    x = inputs.make_x(256, 12)
    W = gemv.weight_matrix(L)
    xt = np.concatenate([_sylvester_pm(128) @ (xb * sb) / SQ for xb, sb in zip(
        np.split(x.view(np.float16).astype(np.float64), 2),
        np.split(1 - 2 * ((L.sign_in[np.arange(256) // 32] >> (np.arange(256) % 32)) & 1).astype(float), 2))])
    yt = fp16.value(L.scales) * (W @ xt)
    y = gemv.gemv(L, x)
    for b in range(2):
        assert np.isclose(np.linalg.norm(y[128 * b:128 * b + 128]), np.linalg.norm(yt[128 * b:128 * b + 128]))


def test_rows_batched_grouped_reduce_to_single_vector():
    L = inputs.make_layer(384, 256, 2, 13)
    X = inputs.make_x(256, 13, rows=3)
    y0 = gemv.gemv(L, X[1])
    rows = np.array([0, 1, 127, 128, 300, 383])
    assert np.allclose(gemv.gemv_rows(L, X[1], rows), y0[rows], rtol=0, atol=1e-12)
    Y = gemv.gemm(L, X)
    assert np.array_equal(Y[1], y0)
    L2 = inputs.make_layer(128, 256, 1, 14)
    out = gemv.grouped([L, L2], [1, 0], X[0], shared_x=True)
    assert np.array_equal(out[1], gemv.gemv(L, X[0])) and np.array_equal(out[0], gemv.gemv(L2, X[0]))


def _pair_hand(state):
    for row in golden_rows("pair_code_hand_values.txt"):
        if int(row[0], 16) == state:
            return (float(np.array([int(row[5], 16)], np.uint16).view(np.float16)[0]),
                    float(np.array([int(row[8], 16)], np.uint16).view(np.float16)[0]))
    raise KeyError(state)


def test_pair_code_all_zero_stream_closed_form():
    """Pair code, all-zero stream: even columns hold w_e = code(0) even weight, odd columns w_o.
    Per input block, the even entries of H v sum to 64 (v_0 + v_1) / sqrt(128) and the odd
    ones to 64 (v_0 - v_1) / sqrt(128), so with g = 1 every row of y~ is
        c = sum_b 64/sqrt(128) * (w_e (v_b0 + v_b1) + w_o (v_b0 - v_b1)),  v = s_in * x,
    and y_o = s_out[o] * c * sqrt(128) for o = 0 mod 128, 0 otherwise."""
    m, n, k = 256, 384, 3
    L = _layer(m, n, k, codes=np.zeros(inputs.words_per_layer(m, n, k), np.uint32),
               scales=_bits(np.ones(m)))
    L.code_id = 1
    x = inputs.make_x(n, 21)
    we, wo = _pair_hand(0)
    s_in = 1 - 2 * ((L.sign_in[np.arange(n) // 32] >> (np.arange(n) % 32)) & 1).astype(np.float64)
    s_out = 1 - 2 * ((L.sign_out[np.arange(m) // 32] >> (np.arange(m) % 32)) & 1).astype(np.float64)
    v = s_in * x.view(np.float16).astype(np.float64)
    c = sum(64 / SQ * (we * (v[128 * b] + v[128 * b + 1]) + wo * (v[128 * b] - v[128 * b + 1]))
            for b in range(n // 128))
    expect = np.zeros(m)
    expect[::128] = s_out[::128] * c * SQ
    y = gemv.gemv(L, x)
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-12 * np.abs(expect).max())


def test_pair_code_tile_layout():
    """Pair code: one all-ones tile gives alternating (even, odd) weights of state 0xFFFF there."""
    m, n, k = 128, 256, 2
    codes = np.zeros(inputs.words_per_layer(m, n, k), np.uint32)
    R, C = 3, 9
    T = R * (n // 16) + C
    codes[T * 8 * k:(T + 1) * 8 * k] = 0xFFFFFFFF
    L = _layer(m, n, k, codes=codes)
    L.code_id = 1
    W = gemv.decode_layer(L)
    e0, o0 = _pair_hand(0)
    e1, o1 = _pair_hand(0xFFFF)
    expect = np.tile(_bits([e0, o0]), (m, n // 2))
    expect[16 * R:16 * R + 16, 16 * C:16 * C + 16] = np.tile(_bits([e1, o1]), (16, 8))
    assert np.array_equal(W, expect)


def test_naive_triple_loop_small_layer():
    """The 256x256 K=2 layer by plain Python loops over every element: signs and the
    (-1)^popcount(i & j) / sqrt(128) Hadamard entries on the input side, the scaled
    product with the decoded weights, then the Hadamard entries and signs on the output
    side -- against the oracle's NumPy route."""
    wl = inputs.CFG1
    m, n, k = wl.tensors["linear"]
    L = inputs.make_layer(m, n, k, wl.seed)
    x = inputs.make_x(n, wl.seed)
    W = gemv.weight_matrix(L).tolist()
    xv = [float(v) for v in x.view(np.float16)]
    g = [float(v) for v in L.scales.view(np.float16)]
    sin = [-1.0 if (int(L.sign_in[i // 32]) >> (i % 32)) & 1 else 1.0 for i in range(n)]
    sout = [-1.0 if (int(L.sign_out[o // 32]) >> (o % 32)) & 1 else 1.0 for o in range(m)]
    r = 1.0 / 128 ** 0.5
    xt = [0.0] * n
    for i in range(n):
        b = i - i % 128
        xt[i] = sum((-1.0 if bin((i % 128) & j).count("1") % 2 else 1.0) * sin[b + j] * xv[b + j]
                    for j in range(128)) * r
    yt = [g[o] * sum(W[o][i] * xt[i] for i in range(n)) for o in range(m)]
    y = [0.0] * m
    for o in range(m):
        b = o - o % 128
        y[o] = sout[o] * r * sum((-1.0 if bin((o % 128) & j).count("1") % 2 else 1.0) * yt[b + j]
                                 for j in range(128))
    ref = gemv.gemv(L, x)
    assert np.allclose(ref, y, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_mcg_decode_uses_the_multiply_only_code():
    """code_id 3 (MCG): an all-zero stream decodes to the fixed point's weight 1/4 everywhere;
    one all-ones tile holds the weight of state 0xFFFF -- both from the hand-worked fixture."""
    m, n, k = 128, 256, 2
    codes = np.zeros(inputs.words_per_layer(m, n, k), np.uint32)
    R, C = 5, 11
    T = R * (n // 16) + C
    codes[T * 8 * k:(T + 1) * 8 * k] = 0xFFFFFFFF
    L = _layer(m, n, k, codes=codes)
    L.code_id = 3
    hand = {int(r[0], 16): int(r[7], 16) for r in golden_rows("mcg_hand_values.txt")}
    expect = np.full((m, n), hand[0], np.uint16)
    expect[16 * R:16 * R + 16, 16 * C:16 * C + 16] = hand[0xFFFF]
    assert np.array_equal(gemv.decode_layer(L), expect)
    assert float(np.array([hand[0]], np.uint16).view(np.float16)[0]) == 0.25

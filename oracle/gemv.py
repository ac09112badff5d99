"""The trellis-coded matrix-vector product, in float64 (test infrastructure).

What the path computes ([DD] Section 2 equations; [TQ] Parts eight, nine,
eleven; [FG] "out_scales always"):

    W^[o, i] = code(S_t) of tile (o // 16, i // 16), t = 16 (o % 16) + (i % 16)
               (code_id 1: weights t = 2 tau, 2 tau + 1 share the state S_tau)
    x~ = blockdiag(H_128) diag(s_in) x
    y~ = diag(g) W^ x~                          (g: per-output fp16 scale)
    y  = diag(s_out) blockdiag(H_128) y~

Reading where the pages leave it open: the per-output scale g acts in the rotated
domain, on y~ before the output transform.

Two routes are provided and pinned against each other: the factored route
(transform x, multiply, transform back) and the dense route, which forms
W_eff = diag(s_out) H diag(g) W^ H diag(s_in) and multiplies once. The
batched and grouped forms run the single-vector routine row by row and expert
by expert. Further pins: the all-zero stream has a closed-form output, a
naive Python loop over every element agrees on the 256x256 layer
(tests/test_oracle_gemv.py), unit impulses read out columns.
"""
from __future__ import annotations

import numpy as np

from . import code, fp16, hadamard, trellis


def decode_layer(layer, tile_rows=None) -> np.ndarray:
    """fp16 bit patterns of the decoded weights, [m, n] (or only the listed tile rows).

    code_id 0, 2 and 3: one state per weight. code_id 1: one state per pair of
    weights (t = 2*tau, 2*tau + 1 of the row-major tile order).
    """
    cid = int(getattr(layer, "code_id", 0))
    v = code.CODE_V[cid]
    states = trellis.layer_states(layer.codes, layer.m, layer.n, layer.k_bits, tile_rows, v)
    if cid == 0:
        w = code.weight_bits(states)
    elif cid == 2:
        w = code.mul1_bits(states)
    elif cid == 3:
        w = code.mcg_weight_bits(states)
    else:
        even, odd = code.pair_weight_bits(states)
        w = np.stack([even, odd], axis=-1).reshape(*states.shape[:-1], trellis.SEQ)
    return trellis.states_to_matrix(w).astype(np.uint16)


def weight_matrix(layer, tile_rows=None) -> np.ndarray:
    """Decoded weights W^ as exact float64 values."""
    return fp16.value(decode_layer(layer, tile_rows))


def scales(layer) -> np.ndarray:
    return fp16.value(layer.scales)


def gemv_with_weights(layer, W: np.ndarray, x_bits: np.ndarray) -> np.ndarray:
    """Factored route for one activation vector, given the decoded weights."""
    x = fp16.value(x_bits)
    xt = hadamard.rht_forward(x, layer.sign_in)
    yt = scales(layer) * (W @ xt)
    return hadamard.rht_inverse(yt, layer.sign_out)


def gemv(layer, x_bits: np.ndarray) -> np.ndarray:
    """y = W x for one fp16 activation vector x (given as bit patterns), float64 [m]."""
    return gemv_with_weights(layer, weight_matrix(layer), x_bits)


def effective_matrix(layer, W: np.ndarray = None) -> np.ndarray:
    """Dense route: W_eff = diag(s_out) blockdiag(H) diag(g) W^ blockdiag(H) diag(s_in)."""
    if W is None:
        W = weight_matrix(layer)
    Hm = hadamard.blockdiag_matrix(layer.m)
    Hn = hadamard.blockdiag_matrix(layer.n)
    s_out = hadamard.signs(layer.sign_out, layer.m)
    s_in = hadamard.signs(layer.sign_in, layer.n)
    return (s_out[:, None] * Hm) @ (scales(layer)[:, None] * W) @ (Hn * s_in[None, :])


def gemv_dense(layer, x_bits: np.ndarray) -> np.ndarray:
    return effective_matrix(layer) @ fp16.value(x_bits)


def gemv_rows(layer, x_bits: np.ndarray, rows) -> np.ndarray:
    """y at the listed output indices only, decoding just the 128-row blocks they fall in.

    x_bits is one vector [n] (result [len(rows)]) or a batch [M, n] (result [M, len(rows)]);
    each 128-row block is decoded once and applied to every vector of the batch.
    """
    rows = np.asarray(rows)
    x = fp16.value(x_bits)
    xt = hadamard.rht_forward(x, layer.sign_in)
    g = scales(layer)
    s_out = hadamard.signs(layer.sign_out, layer.m)
    out = np.empty(x.shape[:-1] + (len(rows),))
    for blk in np.unique(rows // hadamard.BLOCK):
        tr = np.arange(blk * 8, blk * 8 + 8)                      # 8 tile rows = 128 outputs
        W = weight_matrix(layer, tr)
        o = slice(blk * hadamard.BLOCK, (blk + 1) * hadamard.BLOCK)
        yt = g[o] * (xt @ W.T)                                    # W^ x~ for every vector
        yb = s_out[o] * hadamard.apply_blocks(yt)
        sel = rows // hadamard.BLOCK == blk
        out[..., sel] = yb[..., rows[sel] % hadamard.BLOCK]
    return out


# ---------------------------------------------------------------------------
# int8 activations ([TQ] Part eleven: with the mul1 code and activations held
# as int8, decoding a weight and multiplying it fuse into one four-byte dot
# product). The pages fix neither the quantiser nor its scale. Reading, chosen
# so that the integer decision is exact and identical on every machine:
#   u   = blockdiag(+-1 Hadamard) diag(s_in) x     exact in float64 (binary16 x)
#   e_b = the smallest integer with max_{j in block b} |u_j| * 2^-e_b <= 127
#         (e_b = 0 for an all-zero block)
#   q_j = round-half-even(u_j * 2^-e_b)             in -127..127, exact scaling
#   x^_j = q_j * 2^e_b / sqrt(128)                  replaces x~ in y~ = g * (W^ x~)
# Pins (tests/test_oracle_int8.py): the quantiser against a pure-Python route
# with exact fractions and Python's round(); lossless cases (integer u with
# max |u| <= 127) where the int8 product equals the plain GEMV; the half-step
# error bound; every block's largest |q| in 64..127.
# ---------------------------------------------------------------------------

INT8_MAX = 127


def block_exponents(u: np.ndarray) -> np.ndarray:
    """e_b per 128-block of u (last axis): smallest e with max|u_b| 2^-e <= 127."""
    amax = np.abs(hadamard._blocks(u)).max(axis=-1)
    e = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    _, E = np.frexp(amax[nz])                 # amax = f 2^E, f in [1/2, 1): a first guess
    ez = E.astype(np.int64) - 7
    a = amax[nz]
    while True:                               # raise e until the block fits ...
        up = a * np.exp2(-ez.astype(np.float64)) > INT8_MAX
        if not up.any():
            break
        ez += up
    while True:                               # ... and lower it while it still fits
        down = a * np.exp2(-(ez - 1).astype(np.float64)) <= INT8_MAX
        if not down.any():
            break
        ez -= down
    e[nz] = ez
    return e


def quantize_rotated(layer, x_bits: np.ndarray):
    """(q int64 [..., n], e int64 [..., n/128]) of the int8 form of x~ for one layer's input signs."""
    x = fp16.value(x_bits)
    u = hadamard.apply_blocks_pm1(hadamard.signs(layer.sign_in, layer.n) * x)
    e = block_exponents(u)
    step = np.repeat(np.exp2(e.astype(np.float64)), hadamard.BLOCK, axis=-1)
    q = np.rint(u / step).astype(np.int64)        # exact scaling by a power of two; rint: ties to even
    return q, e


def dequantized(q: np.ndarray, e: np.ndarray) -> np.ndarray:
    """x^ = q 2^e / sqrt(128), float64."""
    step = np.repeat(np.exp2(e.astype(np.float64)), hadamard.BLOCK, axis=-1)
    return q * step / np.sqrt(hadamard.BLOCK)


def gemv_int8_rows(layer, x_bits: np.ndarray, rows) -> np.ndarray:
    """int8-activation product at the listed outputs: y~ = g * (W^ x^), then the output transform."""
    rows = np.asarray(rows)
    xh = dequantized(*quantize_rotated(layer, x_bits))
    g = scales(layer)
    s_out = hadamard.signs(layer.sign_out, layer.m)
    out = np.empty(xh.shape[:-1] + (len(rows),))
    for blk in np.unique(rows // hadamard.BLOCK):
        W = weight_matrix(layer, np.arange(blk * 8, blk * 8 + 8))
        o = slice(blk * hadamard.BLOCK, (blk + 1) * hadamard.BLOCK)
        yb = s_out[o] * hadamard.apply_blocks(g[o] * (xh @ W.T))
        sel = rows // hadamard.BLOCK == blk
        out[..., sel] = yb[..., rows[sel] % hadamard.BLOCK]
    return out


def gemv_int8(layer, x_bits: np.ndarray) -> np.ndarray:
    """int8-activation product for one vector, all m outputs (the factored route with x^ for x~)."""
    xh = dequantized(*quantize_rotated(layer, x_bits))
    return hadamard.rht_inverse(scales(layer) * (weight_matrix(layer) @ xh), layer.sign_out)


def gemm(layer, X_bits: np.ndarray, W: np.ndarray = None) -> np.ndarray:
    """Batched form, row by row with the single-vector routine. X [M, n] -> Y [M, m]."""
    if W is None:
        W = weight_matrix(layer)
    return np.stack([gemv_with_weights(layer, W, X_bits[i]) for i in range(X_bits.shape[0])])


def gemm_rows(layer, X_bits: np.ndarray, rows) -> np.ndarray:
    """Batched form at sampled output indices. X [M, n] -> [M, len(rows)]."""
    return gemv_rows(layer, np.asarray(X_bits).reshape(-1, layer.n), rows)


def grouped(layers, sel, X_bits: np.ndarray, shared_x: bool) -> list:
    """Grouped form: for each selected layer index, one GEMV (expert by expert).

    shared_x: every selected layer reads the same vector X_bits [n]; otherwise
    X_bits[e] is the input of the e-th selection.
    """
    out = []
    for e, li in enumerate(sel):
        x = X_bits if shared_x else X_bits[e]
        out.append(gemv(layers[int(li)], x))
    return out

"""Mixture-of-experts block over trellis-coded experts (test infrastructure).

    y = sum_i  w_i * down_{e_i}( fp16( silu(gate_{e_i}(x)) * up_{e_i}(x) ) )

for the token's selected experts e_i with router weights w_i. The pages name
mixture-of-experts models and expert parallelism ([DD] Section 4; [TQ] Part
eleven: per-tensor bit widths, experts at their own K) but not the block's
arithmetic. Readings where the pages leave it open: each expert is a gated MLP with the
SiLU gate, silu(v) = v / (1 + exp(-v)); the down projection's input is the
product rounded once to binary16 (every GEMV of this library takes fp16
inputs); the router weights are given per token and combined in selection
order. Every GEMV is the oracle's single-vector routine (gemv.py).

Pins (tests/test_oracle_moe.py): silu's closed forms and symmetry; a closed
form of the whole block on all-zero streams (every projection is then non-zero
only at outputs 0 mod 128, so h and y follow by hand, with silu from SciPy's
logistic function and binary16 rounding from NumPy's cast), which fails if gate
and up are swapped, if silu acts on up, or if h is not rounded to binary16 once;
the block is linear in the router weights and invariant to reordering the
selection.
"""
from __future__ import annotations

import numpy as np

from . import fp16, gemv


def silu(v):
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def expert_hidden(gate_layer, up_layer, x_bits) -> np.ndarray:
    """fp16 bits of silu(gate(x)) * up(x): the down projection's input."""
    return fp16.round_rne(silu(gemv.gemv(gate_layer, x_bits)) * gemv.gemv(up_layer, x_bits))


def moe_block(gate_up_layers, down_layers, sel, weights, x_bits) -> np.ndarray:
    """gate_up_layers[2e], [2e+1] = gate, up of expert e; down_layers[e]. Returns float64 [hidden]."""
    y = None
    for w, e in zip(weights, sel):
        e = int(e)
        h = expert_hidden(gate_up_layers[2 * e], gate_up_layers[2 * e + 1], x_bits)
        part = float(w) * gemv.gemv(down_layers[e], h)
        y = part if y is None else y + part
    return y

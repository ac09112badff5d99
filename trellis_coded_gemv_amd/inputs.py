"""Seeded synthetic inputs shared by the HIP path, its tests, the bench and the oracle.

This module draws random numbers and packs them into the storage formats the
library consumes. It holds none of the method's arithmetic: no trellis
stepping, no code function, no Hadamard transform. Both the CPU oracle and the
GPU path receive the arrays produced here, bit for bit.

Workloads (synthetic stand-ins for trained layers; no weights or datasets are
used anywhere):

* codes   - uniform random 32-bit words. Every bit string is a valid
            tail-biting bitshift-trellis path, so a uniform stream is a valid
            layer ("Trellis Quantization" lecture, Part eight).
* scales  - per-output fp16 scale drawn from U(0.5, 1.5).
* signs   - uniform random bits, one per row / column (the Rademacher sign
            vectors of the randomized Hadamard transform, "ExLlamaV3 & EXL3
            Deep Dive", Section 2).
* x       - fp16(N(0, 1)) activations.

Streams: ``np.random.SeedSequence([master, tensor, copy, field])`` feeding PCG64.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence

import numpy as np

# field identifiers of the seed sequence
F_CODES, F_SCALES, F_SIGN_IN, F_SIGN_OUT, F_X, F_KBITS, F_ROUTING, F_ROUTER_W = range(8)

TILE = 16            # 16 x 16 weights per trellis sequence
RHT_BLOCK = 128      # Hadamard block along each axis


def _rng(master: int, tensor: int, copy: int, fld: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([master, tensor, copy, fld])))


def words_per_layer(m: int, n: int, k_bits: int) -> int:
    """32-bit words of packed trellis codes: 256*K bits per 16x16 tile."""
    return (m // TILE) * (n // TILE) * 8 * k_bits


@dataclass
class LayerArrays:
    """Host copy of one trellis-coded linear layer (out_features m, in_features n)."""
    m: int
    n: int
    k_bits: int
    codes: np.ndarray      # uint32 [(m/16)*(n/16)*8K], tile-row-major, 8K words per tile
    scales: np.ndarray     # uint16 [m], fp16 bit patterns
    sign_in: np.ndarray    # uint32 [ceil(n/32)], bit i%32 of word i/32 set -> -1
    sign_out: np.ndarray   # uint32 [ceil(m/32)]
    code_id: int = 0

    @property
    def code_bytes(self) -> int:
        return int(self.codes.nbytes)


def make_layer(m: int, n: int, k_bits: int, seed: int, tensor: int = 0, copy: int = 0,
               code_id: int = 0) -> LayerArrays:
    """Random-bitstream layer; the code id only labels how the stream is decoded
    (both codes store 8*K words per 16x16 tile)."""
    codes = _rng(seed, tensor, copy, F_CODES).integers(
        0, 1 << 32, size=words_per_layer(m, n, k_bits), dtype=np.uint32)
    scales = _rng(seed, tensor, copy, F_SCALES).uniform(0.5, 1.5, size=m).astype(np.float16).view(np.uint16)
    sign_in = _rng(seed, tensor, copy, F_SIGN_IN).integers(0, 1 << 32, size=(n + 31) // 32, dtype=np.uint32)
    sign_out = _rng(seed, tensor, copy, F_SIGN_OUT).integers(0, 1 << 32, size=(m + 31) // 32, dtype=np.uint32)
    return LayerArrays(m, n, k_bits, codes, scales, sign_in, sign_out, code_id)


def make_x(n: int, seed: int, tensor: int = 0, copy: int = 0, rows: int = 1) -> np.ndarray:
    """fp16(N(0,1)) activations as uint16 bit patterns, shape [n] (rows == 1) or [rows, n]."""
    x = _rng(seed, tensor, copy, F_X).standard_normal(size=(rows, n)).astype(np.float16).view(np.uint16)
    return x[0] if rows == 1 else x


def draw_kbits(seed: int, tensor: int, choices: Sequence[int]) -> int:
    return int(_rng(seed, tensor, 0, F_KBITS).choice(np.asarray(choices)))


def draw_router_weights(seed: int, tokens: int, top_k: int) -> np.ndarray:
    """Router weights of the selected experts: softmax over top_k N(0,1) logits per token. float32 [tokens, top_k]."""
    logits = _rng(seed, 0, 0, F_ROUTER_W).standard_normal((tokens, top_k))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def draw_routing(seed: int, tokens: int, experts: int, top_k: int) -> np.ndarray:
    """top_k distinct expert indices per token, uniform without replacement. int32 [tokens, top_k]."""
    rng = _rng(seed, 0, 0, F_ROUTING)
    return np.stack([rng.choice(experts, size=top_k, replace=False) for _ in range(tokens)]).astype(np.int32)


# ---------------------------------------------------------------------------
# The five workloads. Shapes are (out_features m, in_features n).
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    seed: int
    tensors: Dict[str, tuple] = field(default_factory=dict)   # name -> (m, n, K)
    batch: int = 1
    note: str = ""


CFG1 = Workload("linear_256x256_k2", 101, {"linear": (256, 256, 2)}, 1,
                "single 256->256 linear, K=2, batch 1")
CFG2 = Workload("llama3_8b_down_14336x4096_k3", 202, {"down": (4096, 14336, 3)}, 1,
                "Llama-3-8B-shaped MLP down-projection 14336->4096, K=3, batch-1 GEMV")
CFG3 = Workload("decoder70b_layer_k2", 303, {
    "q": (8192, 8192, 2), "k": (1024, 8192, 2), "v": (1024, 8192, 2), "o": (8192, 8192, 2),
    "gate": (28672, 8192, 2), "up": (28672, 8192, 2), "down": (8192, 28672, 2)}, 1,
    "all seven linears of one 70B-shaped decoder layer, K=2, batch 1")
CFG4 = Workload("gate_8192x28672_k4_m16", 404, {"gate": (28672, 8192, 4)}, 16,
                "gate projection 8192->28672, K=4, 16 activation rows (MFMA path)")
PREFILL = Workload("prefill_gate_8192x28672_k4_m512", 606, {"gate": (28672, 8192, 4)}, 512,
                   "gate projection 8192->28672, K=4, 512 activation rows (decode into the matrix-core operands)")


@dataclass
class MoEWorkload:
    name: str = "moe_128x_2048_768_k123_top8"
    seed: int = 505
    experts: int = 128
    hidden: int = 2048
    inter: int = 768
    top_k: int = 8
    k_choices: tuple = (1, 2, 3)
    tokens: int = 64

    def tensor_index(self, expert: int, which: str) -> int:
        return 3 * expert + {"gate": 0, "up": 1, "down": 2}[which]

    def shape(self, which: str) -> tuple:
        return (self.inter, self.hidden) if which in ("gate", "up") else (self.hidden, self.inter)

    def kbits(self, expert: int, which: str) -> int:
        return draw_kbits(self.seed, self.tensor_index(expert, which), self.k_choices)

    def layer(self, expert: int, which: str, copy: int = 0, code_id: int = 0) -> LayerArrays:
        m, n = self.shape(which)
        return make_layer(m, n, self.kbits(expert, which), self.seed, self.tensor_index(expert, which), copy,
                          code_id)

    def all_layers(self, copy: int = 0, code_id: int = 0) -> List[LayerArrays]:
        return [self.layer(e, w, copy, code_id) for e in range(self.experts) for w in ("gate", "up", "down")]

    def routing(self) -> np.ndarray:
        return draw_routing(self.seed, self.tokens, self.experts, self.top_k)

    def router_weights(self) -> np.ndarray:
        return draw_router_weights(self.seed, self.tokens, self.top_k)


CFG5 = MoEWorkload()

WORKLOADS = {1: CFG1, 2: CFG2, 3: CFG3, 4: CFG4, 5: CFG5, 6: PREFILL}

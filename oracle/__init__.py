"""CPU oracle for the trellis-coded GEMV -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

A plain, slow, obviously correct NumPy implementation of what the hot path
computes: it walks each tile's bitstream state by state, evaluates the computed
code, builds the full weight matrix, applies explicit +-1 sign vectors and
explicit normalised 128-point Hadamard blocks, and does the matrix-vector
product in float64.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package. The library
(``trellis_coded_gemv_amd``) never imports it, and this package imports nothing
from the library: the two share only the seeded input arrays.

Sources (web pages on QTIP / EXL3 trellis quantization):
  [DD]  "ExLlamaV3 & EXL3 Deep Dive" -- Section 2 (randomized Hadamard
        incoherence equations), Section 3 (bitshift-trellis transition equation
        and the L=12, b=2 state-shift figure).
  [TQ]  "Trellis Quantization: Trading Memory for Cheap Compute" (lecture) --
        Part three (mantissa-splice int->fp16 trick), Part eight (16-bit window,
        random access at bit K*t, 16x16 tiles, tail-biting circle), Part nine
        (3INST computed code), Part eleven (EXL3: 128-blocks, K from 1 to 8,
        the MCG and mul1 codes, int8 activations fused into the four-byte dot
        product), Part twelve (the masked byte-sum integer generator).
  [FG]  "LLM Cal" EXL3 field guide -- "What QTIP contributes" (16x16 block as
        one sequence, tail-biting), "out_scales always", "What the EXL3
        converter actually sets" (mul1 is the default codebook).

Parity status of each function (what pins it, beyond itself) is listed in the
module docstrings. Functions whose end-to-end values have no printed worked
example on the pages are pinned by closed forms, invariants, brute force and
hand-derived values instead; none is "parity unpinned".
"""
from . import fp16, trellis, code, hadamard, gemv  # noqa: F401

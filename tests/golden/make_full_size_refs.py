"""Write the oracle's outputs for the full-size parity tests: tests/golden/full_size_refs.npz.

    python tests/golden/make_full_size_refs.py [--jobs 8] [--reuse]

Every case is a full-size layer of one of the workloads (seeded inputs from
trellis_coded_gemv_amd/inputs.py); the stored values are the oracle's y at two
outputs of every 128-output block (each block has its own split-K handoff in the
GPU kernels), for the activation rows the test checks. The values come from
oracle/ only (oracle.gemv.gemv_rows / gemm_rows). Decoding a whole large layer in
the oracle takes about a minute, too long inside a GPU test, hence the file.
The GPU tests regenerate the same inputs from the same seeds and compare.
Cases marked int8 hold the oracle's int8-activation product of the mul1 code
(oracle.gemv.gemv_int8_rows). --reuse keeps the stored outputs of cases whose
description is unchanged and computes only the others.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "full_size_refs.npz")


def sample_rows(m, seed=0, per_block=2):
    """per_block random outputs in every 128-output block."""
    rng = np.random.default_rng(seed)
    rows = [128 * b + np.sort(rng.choice(128, per_block, replace=False)) for b in range(m // 128)]
    return np.concatenate(rows)


def _cases():
    """key -> case. x: (seed, tensor, rows); pick: activation rows checked (None = all)."""
    sys.path.insert(0, ROOT)
    from trellis_coded_gemv_amd import inputs
    cases = {}
    for cfg, code_ids in ((2, (0, 1)), (3, (0, 3))):
        wl = inputs.WORKLOADS[cfg]
        for ti, (name, (m, n, k)) in enumerate(wl.tensors.items()):
            for cid in code_ids:
                cases[f"w{cfg}_{name}_c{cid}"] = dict(m=m, n=n, k=k, seed=wl.seed, tensor=ti, code_id=cid,
                                                     x=(wl.seed, ti, 1), pick=None, sample_seed=ti)
    for ti, name in ((1, "k"), (4, "gate"), (6, "down")):
        m, n, k = inputs.CFG3.tensors[name]
        cases[f"w3_{name}_c1"] = dict(m=m, n=n, k=k, seed=inputs.CFG3.seed, tensor=ti, code_id=1,
                                      x=(inputs.CFG3.seed, ti, 1), pick=None, sample_seed=ti)
    # the fused launches of the decoder layer: q/k/v read one shared vector, gate/up another
    for cid, names in ((0, ("q", "k", "v", "gate", "up")), (1, ("q", "k", "v")), (3, ("q", "k", "v", "gate", "up"))):
        for name in names:
            ti = list(inputs.CFG3.tensors).index(name)
            m, n, k = inputs.CFG3.tensors[name]
            shared = 100 if name in ("q", "k", "v") else 101
            cases[f"w3f_{name}_c{cid}"] = dict(m=m, n=n, k=k, seed=inputs.CFG3.seed, tensor=ti, code_id=cid,
                                              x=(inputs.CFG3.seed, shared, 1), pick=None, sample_seed=ti)
    # mul1 (code_id 2) with int8 activations: every layer of the decoder layer, q/k/v and gate/up
    # on their shared vectors as in the fused launches, o and down on their own
    for ti, name in enumerate(inputs.CFG3.tensors):
        m, n, k = inputs.CFG3.tensors[name]
        shared = {"q": 100, "k": 100, "v": 100, "gate": 101, "up": 101}.get(name, ti)
        cases[f"w3i8_{name}_c2"] = dict(m=m, n=n, k=k, seed=inputs.CFG3.seed, tensor=ti, code_id=2,
                                         x=(inputs.CFG3.seed, shared, 1), pick=None, sample_seed=ti, int8=True)
    m, n, k = inputs.CFG3.tensors["down"]
    cases["w3_down_c2"] = dict(m=m, n=n, k=k, seed=inputs.CFG3.seed, tensor=6, code_id=2,
                               x=(inputs.CFG3.seed, 6, 1), pick=None, sample_seed=6)
    m, n, k = inputs.CFG4.tensors["gate"]
    for cid in (0, 1, 2, 3):
        cases[f"w4_gate_c{cid}"] = dict(m=m, n=n, k=k, seed=inputs.CFG4.seed, tensor=0, code_id=cid,
                                        x=(inputs.CFG4.seed, 0, inputs.CFG4.batch), pick=None, sample_seed=4)
    cases["prefill_gate_m256_c0"] = dict(m=m, n=n, k=k, seed=inputs.CFG4.seed, tensor=0, code_id=0,
                                         x=(inputs.CFG4.seed, 0, 256), pick=[0, 100, 255], sample_seed=6)
    cases["slots_32768x4096_c0"] = dict(m=32768, n=4096, k=2, seed=96, tensor=0, code_id=0, x=(96, 0, 1),
                                        pick=None, sample_seed=0)
    return cases


CASES = _cases()


def case_inputs(key):
    """(layer arrays, x bits [n] or [M, n], sampled output rows, checked activation rows or None)."""
    from trellis_coded_gemv_amd import inputs
    c = CASES[key]
    arr = inputs.make_layer(c["m"], c["n"], c["k"], c["seed"], tensor=c["tensor"], code_id=c["code_id"])
    xs, xt, rows = c["x"]
    X = inputs.make_x(c["n"], xs, tensor=xt, rows=rows)
    return arr, X, sample_rows(c["m"], seed=c["sample_seed"]), c["pick"]


def _compute(key):
    from oracle import gemv
    arr, X, rows, pick = case_inputs(key)
    if CASES[key].get("int8"):
        return key, rows, gemv.gemv_int8_rows(arr, X, rows)[None, :]
    if X.ndim == 1:
        y = gemv.gemv_rows(arr, X, rows)[None, :]
    else:
        y = gemv.gemm_rows(arr, X if pick is None else X[pick], rows)
    return key, rows, y


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--reuse", action="store_true")
    args = ap.parse_args(argv)
    keep = {}
    if args.reuse and os.path.exists(OUT):
        z = np.load(OUT, allow_pickle=False)
        old = json.loads(str(z["meta"]))
        for key in CASES:
            if old.get(key) == json.loads(json.dumps(CASES[key])):
                keep[key] = (key, z[key + "/rows"], z[key + "/y"])
    import multiprocessing as mp
    todo = sorted(k for k in CASES if k not in keep)
    with mp.get_context("fork").Pool(args.jobs) as pool:
        res = pool.map(_compute, todo, chunksize=1) + list(keep.values())
    out = {"meta": np.array(json.dumps(CASES, sort_keys=True))}
    for key, rows, y in res:
        out[key + "/rows"] = rows.astype(np.int32)
        out[key + "/y"] = y
        print(key, y.shape, flush=True)
    np.savez_compressed(OUT, **out)
    print("wrote", OUT)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the trellis-coded GEMV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

A step is one pass of the whole hot path over one batch of synthetic input:
input-side randomized Hadamard transform, trellis decode of every weight,
dot products, split-K reduction, per-output scale and output-side transform,
through the C ABI. Workloads (seeded, synthetic; no trained weights):

  1  one 256x256 linear, K=2, batch 1
  2  Llama-3-8B-shaped MLP down-projection 14336 -> 4096, K=3, batch 1 (default)
  3  the seven linears of a 70B-shaped decoder layer, K=2, batch 1 (a step = 7 GEMVs)
  4  gate projection 8192 -> 28672, K=4, 16 activation rows (MFMA path)
  5  MoE: 128 experts (gate/up 2048->768, down 768->2048, K in {1,2,3}), top-8 per
     token, a step = one token = 2 grouped launches
  6  prefill: gate projection 8192 -> 28672, K=4, 512 activation rows (decode once
     to fp16 + dense GEMM; its roofline is the matrix cores')
  7  the workload-5 experts as a whole MoE block per token: gate/up -> silu * mul ->
     down -> router-weighted combine (3 launches)

Enough seeded copies of the weights (>= 1 GiB, four times the 256 MB Infinity
Cache) are used round-robin that the timed reads come from HBM. Inputs are in
device memory before the timed region starts.

Prints ONE JSON line: value = compressed-weight GB/s over the timed region (K
steps between two synchronisations, HIP events on the launch stream, steps
replayed from a captured HIP graph), the roofline of the dominant kernel, and
the CPU oracle timed on a bounded sample of the same workload on the host.

The dominant kernel (the launch moving the most bytes) is timed alone: the same
K steps restricted to its launches, replayed from their own graph, give its mean
launch duration. The decode is bound by VALU arithmetic, so the roofline is an
ALU one: algorithmic lane-operations per launch (decoded weights x the minimum
VALU operations per weight the code needs on gfx950: window extract,
multiply-add, and-or, dot2 = 4 for code 0; 2 for the pair code, one state per
two weights; one fewer per state on the MFMA path, whose dot products run on
the matrix cores) over the launch duration, against 256 CUs x 4 SIMDs x 16
lanes x 2.4 GHz = 39.3 T lane-operations/s. The same launch's HBM view
(algorithmic bytes / duration against 8 TB/s) and the measured HBM traffic
(rocprofv3 FETCH_SIZE + WRITE_SIZE, profiles/traffic.json) are reported with it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "batch-1 trellis GEMV: compressed-weight HBM GB/s (% of peak) + µs/layer"
HBM_PEAK_GBS = 8000.0
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12      # VALU lane-operations per second, in T (39.32)
MFMA_F16_PEAK_TFLOPS = 2500.0
CACHE_DEFEAT_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    """Hash of the HIP sources: counter-derived traffic is only reported for the kernels it was taken on."""
    import hashlib
    d = os.path.join(ROOT, "trellis_coded_gemv_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: int, kernel: str, code_id: int = 0):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("csrc_sha") != kernel_source_hash():
        return None
    key = str(workload) if code_id == 0 else f"{workload}/code{code_id}"
    ent = rec.get("workloads", {}).get(key, {}).get(kernel)
    return None if ent is None else int(ent["hbm_bytes_per_launch"])


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def alu_ops_per_weight(code_id: int, mfma: bool) -> float:
    """Minimum VALU lane-operations per decoded weight (see the module docstring)."""
    per_state = 3 if mfma else 4          # window extract, multiply-add, and-or (+ dot2 on the VALU path)
    return per_state / (2 if code_id == 1 else 1)


def gemv_bytes(m: int, n: int, k: int, M: int = 1) -> int:
    """Algorithmic bytes of one layer call: codes + x (fp16) + y (fp32) + scales (fp16) + sign bits."""
    return m * n * k // 8 + 2 * n * M + 4 * m * M + 2 * m + (n + m) // 8


class Launches:
    """Runs the launches of a step; `only` restricts a pass to one kernel (for its own timing)."""

    def __init__(self, only=None):
        self.only = only

    def __call__(self, name, fn):
        if self.only is None or name == self.only:
            fn()


def graph_time_ms(torch, step, steps, launches):
    """Capture `steps` steps into one HIP graph, replay it once between two events; return ms."""
    stream = torch.cuda.current_stream()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(stream)
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                step(i, launches)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b)


# ---------------------------------------------------------------------------
# workloads: each returns (step(i, launches), info) with device data prepared
# ---------------------------------------------------------------------------

MAX_COPIES = 64


def _copies(total_bytes):
    # tiny layers (the 256x256 case) cannot defeat the caches with a sane number of copies:
    # they are latency-bound and their number is reported as such
    return max(1, min(MAX_COPIES, math.ceil(CACHE_DEFEAT_BYTES / total_bytes)))


def setup_linears(torch, tg, inputs, wl, dev, code_id):
    """Workloads 1-3: batch-1 GEMVs over the workload's tensors, one call each per step."""
    names = list(wl.tensors)
    code_bytes = sum(m * n * k // 8 for (m, n, k) in wl.tensors.values())
    copies = _copies(code_bytes)
    log(f"{wl.name}: {len(names)} tensor(s), {code_bytes} code bytes per step, {copies} copies")
    per = []
    for c in range(copies):
        layers = {}
        for ti, name in enumerate(names):
            m, n, k = wl.tensors[name]
            L = tg.DeviceLayer(inputs.make_layer(m, n, k, wl.seed, tensor=ti, copy=c, code_id=code_id), dev)
            x = tg.fp16_tensor(inputs.make_x(n, wl.seed, tensor=ti, copy=c), dev)
            y = torch.empty(m, dtype=torch.float32, device=dev)
            layers[name] = (L, x, y)
        per.append(layers)
    ws = {name: tg.workspace(per[0][name][0], 1, dev) for name in names}

    def step(i, launch):
        layers = per[i % copies]
        for name in names:
            L, x, y = layers[name]
            launch(name, lambda L=L, x=x, y=y, w=ws[name]: tg.trellis_gemv(L, x, y, w, torch.cuda.current_stream()))

    alg = {name: gemv_bytes(*wl.tensors[name]) for name in names}
    return step, dict(code_bytes=code_bytes, copies=copies, alg_bytes=alg, names=names,
                      weights={name: wl.tensors[name][0] * wl.tensors[name][1] for name in names}, mfma=False,
                      units="layer" if len(names) == 1 else "decoder layer (7 GEMVs)")


def setup_gemm(torch, tg, inputs, wl, dev, code_id):
    name = "gate"
    m, n, k = wl.tensors[name]
    M = wl.batch
    code_bytes = m * n * k // 8
    copies = _copies(code_bytes)
    log(f"{wl.name}: M={M}, {code_bytes} code bytes, {copies} copies")
    per = []
    for c in range(copies):
        L = tg.DeviceLayer(inputs.make_layer(m, n, k, wl.seed, tensor=0, copy=c, code_id=code_id), dev)
        X = tg.fp16_tensor(inputs.make_x(n, wl.seed, tensor=0, copy=c, rows=M), dev)
        Y = torch.empty(M, m, dtype=torch.float32, device=dev)
        per.append((L, X, Y))
    ws = tg.workspace(per[0][0], M, dev)

    def step(i, launch):
        L, X, Y = per[i % copies]
        launch(name, lambda: tg.trellis_gemm_small(L, X, Y, ws, torch.cuda.current_stream()))

    return step, dict(code_bytes=code_bytes, copies=copies, alg_bytes={name: gemv_bytes(m, n, k, M)},
                      names=[name], weights={name: m * n}, mfma=True, units="layer (16 rows)",
                      flops=2.0 * m * n * M)


def setup_prefill(torch, tg, inputs, wl, dev, code_id):
    name = "gate"
    m, n, k = wl.tensors[name]
    M = wl.batch
    code_bytes = m * n * k // 8
    copies = _copies(code_bytes)
    log(f"{wl.name}: M={M}, {code_bytes} code bytes, {copies} copies")
    per = []
    for c in range(copies):
        L = tg.DeviceLayer(inputs.make_layer(m, n, k, wl.seed, tensor=0, copy=c, code_id=code_id), dev)
        X = tg.fp16_tensor(inputs.make_x(n, wl.seed, tensor=0, copy=c, rows=M), dev)
        per.append((L, X))
    Y = torch.empty(M, m, dtype=torch.float32, device=dev)
    ws = tg.prefill_workspace(per[0][0], M, dev)

    def step(i, launch):
        L, X = per[i % copies]
        launch(name, lambda: tg.trellis_gemm_prefill(L, X, Y, ws, torch.cuda.current_stream()))

    return step, dict(code_bytes=code_bytes, copies=copies, alg_bytes={name: gemv_bytes(m, n, k, M)},
                      names=[name], weights={name: m * n}, mfma=True, prefill=True,
                      units=f"layer ({M} rows)", flops=2.0 * m * n * M)


def setup_moe_block(torch, tg, inputs, wl, dev, code_id):
    routing, rw = wl.routing(), wl.router_weights()
    gu_arr = [wl.layer(e, w, code_id=code_id) for e in range(wl.experts) for w in ("gate", "up")]
    dn_arr = [wl.layer(e, "down", code_id=code_id) for e in range(wl.experts)]
    all_bytes = sum(a.code_bytes for a in gu_arr + dn_arr)
    copies = _copies(all_bytes)
    log(f"{wl.name} block: {all_bytes} code bytes for all experts, {copies} copies, {wl.tokens} tokens")
    tables = []
    for c in range(copies):
        gu = [tg.DeviceLayer(wl.layer(e, w, copy=c, code_id=code_id), dev) for e in range(wl.experts)
              for w in ("gate", "up")]
        dn = [tg.DeviceLayer(wl.layer(e, "down", copy=c, code_id=code_id), dev) for e in range(wl.experts)]
        tables.append((tg.LayerTable(gu, dev), tg.LayerTable(dn, dev)))
    sels = [torch.tensor(routing[t], dtype=torch.int32, device=dev) for t in range(wl.tokens)]
    wts = [torch.tensor(rw[t], dtype=torch.float32, device=dev) for t in range(wl.tokens)]
    xs = [tg.fp16_tensor(inputs.make_x(wl.hidden, wl.seed, tensor=10_000 + t), dev) for t in range(wl.tokens)]
    y = torch.empty(wl.hidden, dtype=torch.float32, device=dev)
    ws = tg.moe_workspace(tables[0][0], tables[0][1], wl.top_k, dev)
    tok_bytes = [sum(gu_arr[2 * int(e) + w].code_bytes for e in routing[t] for w in (0, 1)) +
                 sum(dn_arr[int(e)].code_bytes for e in routing[t]) for t in range(wl.tokens)]

    def step(i, launch):
        t = i % wl.tokens
        gu_t, dn_t = tables[(i // wl.tokens) % copies]
        s = torch.cuda.current_stream()
        launch("block", lambda: tg.trellis_moe_block(gu_t, dn_t, sels[t], wts[t], xs[t], y, ws, s))

    mean_tok = float(np.mean(tok_bytes))
    k2 = 2 * wl.top_k
    # codes + x (fp16) + y (fp32) + scales (fp16) + the fp32 intermediates, each written once and read once
    alg = {"block": mean_tok + 2 * wl.hidden + 4 * wl.hidden + 2 * (k2 * wl.inter + wl.top_k * wl.hidden) +
           2 * 4 * (k2 * wl.inter + wl.top_k * wl.hidden)}
    return step, dict(code_bytes=mean_tok, copies=copies, alg_bytes=alg, names=["block"],
                      weights={"block": 3 * wl.top_k * wl.inter * wl.hidden}, mfma=False,
                      units="token (MoE block, 3 launches)")


def setup_moe(torch, tg, inputs, wl, dev, code_id):
    routing = wl.routing()
    gu_arr = [wl.layer(e, w, code_id=code_id) for e in range(wl.experts) for w in ("gate", "up")]
    dn_arr = [wl.layer(e, "down", code_id=code_id) for e in range(wl.experts)]
    all_bytes = sum(a.code_bytes for a in gu_arr + dn_arr)
    copies = _copies(all_bytes)
    log(f"{wl.name}: {all_bytes} code bytes for all experts, {copies} copies, {wl.tokens} tokens")
    tables = []
    for c in range(copies):
        gu = [tg.DeviceLayer(wl.layer(e, w, copy=c, code_id=code_id), dev) for e in range(wl.experts) for w in ("gate", "up")]
        dn = [tg.DeviceLayer(wl.layer(e, "down", copy=c, code_id=code_id), dev) for e in range(wl.experts)]
        tables.append((tg.LayerTable(gu, dev), tg.LayerTable(dn, dev)))
    sel_gu = [torch.tensor([2 * int(e) + w for e in routing[t] for w in (0, 1)], dtype=torch.int32, device=dev)
              for t in range(wl.tokens)]
    sel_dn = [torch.tensor([int(e) for e in routing[t]], dtype=torch.int32, device=dev) for t in range(wl.tokens)]
    xs = [tg.fp16_tensor(inputs.make_x(wl.hidden, wl.seed, tensor=10_000 + t), dev) for t in range(wl.tokens)]
    xds = [tg.fp16_tensor(inputs.make_x(wl.inter, wl.seed, tensor=20_000 + t, rows=wl.top_k), dev)
           for t in range(wl.tokens)]
    Y1 = torch.empty(2 * wl.top_k, wl.inter, dtype=torch.float32, device=dev)
    Y2 = torch.empty(wl.top_k, wl.hidden, dtype=torch.float32, device=dev)
    ws1 = tg.grouped_workspace(tables[0][0], 2 * wl.top_k, dev)
    ws2 = tg.grouped_workspace(tables[0][1], wl.top_k, dev)
    tok_bytes = [sum(gu_arr[2 * int(e) + w].code_bytes for e in routing[t] for w in (0, 1)) +
                 sum(dn_arr[int(e)].code_bytes for e in routing[t]) for t in range(wl.tokens)]

    def step(i, launch):
        t = i % wl.tokens
        gu_t, dn_t = tables[(i // wl.tokens) % copies]
        s = torch.cuda.current_stream()
        launch("gate_up", lambda: tg.trellis_gemv_grouped(gu_t, sel_gu[t], xs[t], 0, Y1, wl.inter, ws1, s))
        launch("down", lambda: tg.trellis_gemv_grouped(dn_t, sel_dn[t], xds[t], wl.inter, Y2, wl.hidden, ws2, s))

    mean_tok = float(np.mean(tok_bytes))
    alg = {"gate_up": mean_tok * 2 / 3 + 2 * wl.hidden + 16 * 6 * wl.inter,
           "down": mean_tok / 3 + 8 * 2 * wl.inter + 8 * 6 * wl.hidden}
    return step, dict(code_bytes=mean_tok, copies=copies, alg_bytes=alg, names=["gate_up", "down"],
                      weights={"gate_up": 2 * wl.top_k * wl.inter * wl.hidden, "down": wl.top_k * wl.hidden * wl.inter},
                      mfma=False, units="token (24 GEMVs, 2 launches)")


def run_gpu(workload, steps, warmup, use_graph, code_id=0):
    """Time `steps` steps of the workload. Returns (info, timings).

    region_ms: the timed region (all launches of K steps, graph replay unless disabled).
    dom_ms: the dominant kernel alone -- the same K steps restricted to its launches,
            replayed back to back -- i.e. K times its mean launch duration.
    """
    import torch
    from trellis_coded_gemv_amd import binding as tg
    from trellis_coded_gemv_amd import inputs

    dev = "cuda"
    wl = workload_of(inputs, workload)
    setup = {1: setup_linears, 2: setup_linears, 3: setup_linears, 4: setup_gemm, 5: setup_moe,
             6: setup_prefill, 7: setup_moe_block}[workload]
    step, info = setup(torch, tg, inputs, wl, dev, code_id)
    dom = max(info["names"], key=lambda k: info["alg_bytes"][k])     # kernel moving the most bytes
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i, Launches())
    torch.cuda.synchronize()

    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        step(i, Launches())
    t1.record(stream)
    torch.cuda.synchronize()
    eager_ms = t0.elapsed_time(t1)

    region_ms, dom_ms, timing = eager_ms, None, "eager launches"
    if use_graph:
        try:
            region_ms = graph_time_ms(torch, step, steps, Launches())
            dom_ms = graph_time_ms(torch, step, steps, Launches(only=dom))
            timing = "graph replay"
        except Exception as e:  # noqa: BLE001 - keep the eager number
            log("graph replay unavailable:", repr(e))
    if dom_ms is None:
        t0.record(stream)
        for i in range(steps):
            step(i, Launches(only=dom))
        t1.record(stream)
        torch.cuda.synchronize()
        dom_ms = t0.elapsed_time(t1)
    # Context only, never the metric: the same copy every step (its code words stay in the caches).
    hot_ms = None
    if timing == "graph replay":
        hot_ms = graph_time_ms(torch, lambda i, launches: step(0, launches), steps, Launches())
    return info, dict(region_ms=region_ms, eager_ms=eager_ms, dom=dom, dom_ms=dom_ms, timing=timing, hot_ms=hot_ms,
                      stream_read_gbs=stream_read_gbs(torch))


def stream_read_gbs(torch, nbytes=1 << 30, reps=5):
    """Context: a plain streaming read on the same GPU in the same run (torch.sum over 1 GiB viewed as fp64, the
    fastest read-only library kernel measured here), GB/s, best of reps."""
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(reps + 1):
        a.record()
        buf.view(torch.float64).sum()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None or ms < best else best
    del buf
    return round(nbytes / (best * 1e-3) / 1e9, 1)


def workload_of(inputs, workload):
    """Workload 7 runs the experts of workload 5 as whole MoE blocks."""
    return inputs.WORKLOADS[5 if workload == 7 else workload]


def _moe_token(inputs, wl, code_id, t=0):
    """Token t of the MoE workload: its selected experts' layers (keyed as in the tables), selection, weights, x."""
    sel, w = wl.routing()[t], wl.router_weights()[t]
    gu, dn = {}, {}
    for e in sel:
        e = int(e)
        gu[2 * e], gu[2 * e + 1] = wl.layer(e, "gate", code_id=code_id), wl.layer(e, "up", code_id=code_id)
        dn[e] = wl.layer(e, "down", code_id=code_id)
    return gu, dn, sel, w, inputs.make_x(wl.hidden, wl.seed, tensor=10_000 + t)


def moe_block_parity(inputs, wl, code_id):
    """Token 0 through the whole block (all experts on the device, copy 0) against the oracle's block."""
    import torch
    from oracle import moe
    from trellis_coded_gemv_amd import binding as tg

    gu, dn, sel, w, x = _moe_token(inputs, wl, code_id)
    gut = tg.LayerTable([tg.DeviceLayer(wl.layer(e, k, code_id=code_id), "cuda") for e in range(wl.experts)
                         for k in ("gate", "up")], "cuda")
    dnt = tg.LayerTable([tg.DeviceLayer(wl.layer(e, "down", code_id=code_id), "cuda") for e in range(wl.experts)],
                        "cuda")
    y = tg.trellis_moe_block(gut, dnt, torch.from_numpy(sel).to("cuda"), torch.from_numpy(w).to("cuda"),
                             tg.fp16_tensor(x, "cuda"))
    torch.cuda.synchronize()
    ref = moe.moe_block(gu, dn, sel, w, x)
    return float(np.abs(y.cpu().numpy() - ref).max() / np.abs(ref).max())


def parity_spot_check(workload, code_id=0):
    """Copy 0 of the workload against the oracle on sampled outputs (after timing)."""
    import torch
    from oracle import gemv as ogemv
    from trellis_coded_gemv_amd import binding as tg
    from trellis_coded_gemv_amd import inputs

    wl = workload_of(inputs, workload)
    if workload == 7:
        return moe_block_parity(inputs, wl, code_id)
    if workload == 5:
        e, which = int(wl.routing()[0][0]), "gate"
        arr, x = wl.layer(e, which, code_id=code_id), inputs.make_x(wl.hidden, wl.seed, tensor=10_000)
        rows, M = np.arange(0, wl.inter, 5), 1
    else:
        name = list(wl.tensors)[-1]
        m, n, k = wl.tensors[name]
        ti = list(wl.tensors).index(name)
        arr = inputs.make_layer(m, n, k, wl.seed, tensor=ti, code_id=code_id)
        M = wl.batch
        x = inputs.make_x(n, wl.seed, tensor=ti, rows=M)
        rows = np.concatenate([np.arange(0, 128, 7), np.arange(m - 128, m, 11)])
    L = tg.DeviceLayer(arr, "cuda")
    if M == 1:
        y = tg.trellis_gemv(L, tg.fp16_tensor(x, "cuda"))[None, :]
        ref = ogemv.gemv_rows(arr, x, rows)[None, :]
    elif workload == 6:
        y = tg.trellis_gemm_prefill(L, tg.fp16_tensor(x, "cuda"))
        ref = ogemv.gemm_rows(arr, x[:2], rows)
    else:
        y = tg.trellis_gemm_small(L, tg.fp16_tensor(x, "cuda"))
        ref = ogemv.gemm_rows(arr, x[:2], rows)
    torch.cuda.synchronize()
    y = y.cpu().numpy()[: ref.shape[0], rows]
    return float(np.abs(y - ref).max() / np.abs(ref).max())


def cpu_baseline(workload, sample_blocks, code_id=0):
    """The oracle, untuned, on a bounded sample of the workload, scaled to the same unit (GB/s of codes)."""
    from threadpoolctl import threadpool_limits
    from oracle import gemv as ogemv
    from trellis_coded_gemv_amd import inputs

    wl = workload_of(inputs, workload)
    if workload == 7:
        from oracle import moe
        dt, nbytes, ntok = 0.0, 0, 0
        while ntok < wl.tokens and dt < 10.0:   # whole tokens, about 10 s of oracle work
            gu, dn, sel, w, x = _moe_token(inputs, wl, code_id, ntok)
            with threadpool_limits(limits=1):
                t = time.perf_counter()
                moe.moe_block(gu, dn, sel, w, x)
                dt += time.perf_counter() - t
            nbytes += sum(a.code_bytes for a in list(gu.values()) + list(dn.values()))
            ntok += 1
        sample = f"tokens 0..{ntok - 1}: the whole block over each token's {wl.top_k} experts ({nbytes} code bytes), {dt:.1f} s"
        rate = nbytes / dt
    elif workload == 5:
        arrs = [wl.layer(int(e), w, code_id=code_id) for e in wl.routing()[0][:2] for w in ("gate", "up", "down")]
        xs = [inputs.make_x(a.n, 1) for a in arrs]
        with threadpool_limits(limits=1):
            t = time.perf_counter()
            for a, x in zip(arrs, xs):
                ogemv.gemv(a, x)
            dt = time.perf_counter() - t
        nbytes = sum(a.code_bytes for a in arrs)
        sample = f"gate/up/down of 2 experts (6 full GEMVs, {nbytes} code bytes), {dt:.1f} s"
        rate = nbytes / dt
    else:
        name = max(wl.tensors, key=lambda k: wl.tensors[k][0] * wl.tensors[k][1])
        m, n, k = wl.tensors[name]
        ti = list(wl.tensors).index(name)
        arr = inputs.make_layer(m, n, k, wl.seed, tensor=ti, code_id=code_id)
        M = wl.batch
        Mo = min(M, 16)                        # oracle rows timed; scaled to the M rows of a step
        X = inputs.make_x(n, wl.seed, tensor=ti, rows=Mo) if Mo > 1 else inputs.make_x(n, wl.seed, tensor=ti)
        nb = m // 128
        nblk = max(1, sample_blocks // Mo)
        blocks = np.linspace(0, nb - 1, min(nblk, nb)).astype(int)
        rows = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
        def one_pass():
            if Mo == 1:
                ogemv.gemv_rows(arr, X, rows)
            else:
                ogemv.gemm_rows(arr, X, rows)
        with threadpool_limits(limits=1):
            one_pass()                         # warm-up pass, not timed
            passes, total = 0, 0.0
            while passes < 8 and (passes == 0 or total < 10.0):   # whole passes, about 10 s in all
                t = time.perf_counter()
                one_pass()
                total += time.perf_counter() - t
                passes += 1
        dt = total / passes
        nbytes = len(rows) * n * k // 8
        sample = (f"{len(blocks)} of {nb} 128-output blocks of the {m}x{n} K={k} '{name}' tensor"
                  f"{'' if M == 1 else f' x {Mo} rows'} (decode + fp64 GEMV), {passes} timed pass(es) of {dt:.1f} s"
                  f"{'' if Mo == M else f', scaled to {M} rows'}")
        rate = nbytes / (dt * M / Mo)
    return {"value": round(rate / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle", "sample": sample}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5, 6, 7])
    ap.add_argument("--code", type=int, default=0, choices=[0, 1],
                    help="code_id of every layer: 0 the three-instruction code, 1 the pair code")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--cpu-blocks", type=int, default=32, help="oracle sample size in 128-output blocks (0: skip)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="after timing, write (fill) and read (sum) this many MiB (counter calibration)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library has no multi-GPU path.",
              file=sys.stderr)
        return 2

    from trellis_coded_gemv_amd import inputs
    wl = workload_of(inputs, args.workload)
    info, t = run_gpu(args.workload, args.steps, args.warmup, not args.no_graph, args.code)
    steps = args.steps
    ms_per_step = t["region_ms"] / steps
    value = info["code_bytes"] / (ms_per_step * 1e-3) / 1e9
    dom = t["dom"]
    dom_launch_ms = t["dom_ms"] / steps
    achieved = info["alg_bytes"][dom] / (dom_launch_ms * 1e-3) / 1e9
    opw = alu_ops_per_weight(args.code, info["mfma"])
    alg_ops = info["weights"][dom] * opw
    alu_achieved = alg_ops / (dom_launch_ms * 1e-3) / 1e12
    config = {"workload": wl.name + ("_block" if args.workload == 7 else ""), "units": info["units"], "code_bytes_per_step": int(info["code_bytes"]),
              "copies": info["copies"], "us_per_step": round(ms_per_step * 1e3, 3),
              "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2), "timing": t["timing"],
              "eager_us_per_step": round(t["eager_ms"] / steps * 1e3, 3),
              "context": {"hot_cache_us_per_step": None if t["hot_ms"] is None else round(t["hot_ms"] / steps * 1e3, 3),
                          "stream_read_gbs": t["stream_read_gbs"],
                          "note": "hot: copy 0 every step (caches warm); stream_read: torch.sum over 1 GiB (fp64 view)"},
              "code_id": args.code, "parity_max_rel_err": parity_spot_check(args.workload, args.code)}
    if args.workload not in (5, 7):
        config.update({"tensors": {k: list(v) for k, v in wl.tensors.items()}, "batch": wl.batch})
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16", "data": "synthetic", "config": config,
        "roofline": {"bound": "alu", "kernel": dom, "achieved": round(alu_achieved, 3), "peak": round(ALU_PEAK_TOPS, 3),
                     "unit": "T lane-ops/s", "frac": round(alu_achieved / ALU_PEAK_TOPS, 4),
                     "traffic": recorded_traffic(args.workload, dom, args.code),
                     "algorithmic_ops": int(alg_ops), "ops_per_weight": opw,
                     "launch_us": round(dom_launch_ms * 1e3, 3),
                     "hbm": {"achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(achieved / HBM_PEAK_GBS, 4),
                             "algorithmic_bytes": int(info["alg_bytes"][dom])}},
    }
    if "flops" in info:
        tf = info["flops"] / (dom_launch_ms * 1e-3) / 1e12
        out["roofline"]["mfma"] = {"achieved_tflops": round(tf, 2), "peak_tflops": MFMA_F16_PEAK_TFLOPS,
                                   "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 5)}
    if info.get("prefill"):
        # decode once + dense GEMM: the contraction is the roofline here
        mf = out["roofline"].pop("mfma")
        alu = {k: out["roofline"].pop(k) for k in ("achieved", "peak", "unit", "frac", "algorithmic_ops",
                                                   "ops_per_weight")}
        out["roofline"].update({"bound": "mfma", "achieved": mf["achieved_tflops"], "peak": MFMA_F16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": mf["frac"], "algorithmic_flops": info["flops"],
                                "alu": alu})
    if args.copy_calib_mb > 0:
        # counter calibration: a pure write (fill) and a pure read (sum) of known size
        import torch
        buf = torch.empty(args.copy_calib_mb << 18, dtype=torch.float32, device="cuda")
        for _ in range(3):
            buf.fill_(1.0)
            buf.sum()
        torch.cuda.synchronize()
        out["config"]["calibration_bytes"] = buf.numel() * 4
    if args.cpu_blocks > 0:
        out["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_blocks, args.code)
    out["config"]["csrc_sha"] = kernel_source_hash()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

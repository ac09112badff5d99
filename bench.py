#!/usr/bin/env python3
"""Benchmark of the trellis-coded GEMV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--code 0] [--int8]

A step is one pass of the whole hot path over one batch of synthetic input:
input-side randomized Hadamard transform, trellis decode of every weight,
dot products, split-K reduction, per-output scale and output-side transform,
through the C ABI. Workloads (seeded, synthetic; no trained weights):

  1  one 256x256 linear, K=2, batch 1
  2  Llama-3-8B-shaped MLP down-projection 14336 -> 4096, K=3, batch 1
  3  the seven linears of a 70B-shaped decoder layer, K=2, batch 1 (a step = 7 GEMVs;
     the default: the largest batch-1 workload)
  4  gate projection 8192 -> 28672, K=4, 16 activation rows (MFMA path)
  5  MoE: 128 experts (gate/up 2048->768, down 768->2048, K in {1,2,3}), top-8 per
     token, a step = one token = 2 grouped launches
  6  prefill: gate projection 8192 -> 28672, K=4, 512 activation rows (each weight
     decoded once into the MFMA operands; its roofline is the matrix cores')
  7  the workload-5 experts as a whole MoE block per token: gate/up -> silu * mul ->
     down -> router-weighted combine (3 launches)

Enough seeded copies of the weights (>= 1 GiB, four times the 256 MB Infinity
Cache) are used round-robin, and every timed step uses a copy that at least
1 GiB of other copies were read after, so the timed reads come from HBM.
Inputs are in device memory before the timed region starts.

Prints ONE JSON line: value = compressed-weight GB/s over the timed region (K
steps between two synchronisations, HIP events on the launch stream, steps
replayed from a captured HIP graph), the roofline of the dominant kernel, the
CPU oracle timed on a bounded sample of the same workload on every host core
of the process's affinity mask, and short measurements of workloads 2, 4 and 5
and of the bench's workload with the other codes (MCG, mul1 with int8
activations, the pair code) as context.

Roofline. The dominant launch (the one moving the most bytes) is timed alone:
the same K steps restricted to its launches, replayed from their own graph,
give its mean launch duration. `achieved` = its algorithmic bytes (codes + x
fp16 + y fp32 + scales fp16 + sign bits) / that duration, against the 8 TB/s
HBM peak. The decode is bound by VALU issue in practice, so the line also
carries an ALU view: decoded weights per second of that launch against the
decode-only ceiling (tg_decode_ceiling: the batch-1 loop on code words held
in LDS), measured in the same run. `traffic` is the measured HBM bytes of one
launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, profiles/traffic.json) while the
kernel sources match the ones it was taken on.

--code 2 --int8: the mul1 code with the int8 form of the rotated input (the
batch-1 workloads 1-3; the context workloads then run code 2 without it).
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
MFMA_F16_PEAK_TFLOPS = 2500.0
CACHE_DEFEAT_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
DEFAULT_WORKLOAD = 3


def kernel_source_hash() -> str:
    """Hash of the library sources (the library reports the same value as tg_build_id())."""
    from trellis_coded_gemv_amd.build import source_hash
    return source_hash()


def recorded_traffic(workload: int, kernel: str, code_id: int = 0):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("csrc_sha") != kernel_source_hash():
        return None
    key = str(workload) if code_id == 0 else f"{workload}/code{code_id}"
    if LAYER_FLAGS["int8"]:
        key += "/int8"
    ent = rec.get("workloads", {}).get(key, {}).get(kernel)
    return None if ent is None else int(ent["hbm_bytes_per_launch"])


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


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


def timed_steps_ms(torch, step, first, steps, copies, launches, use_graph):
    """Time `steps` steps starting at step index `first`. Returns (ms, how).

    Graph mode captures the steps into one HIP graph and replays it once untimed; then,
    if the steps use fewer copies than there are, eager steps over the other copies run
    (so each timed copy was last read before at least 1 GiB of other copies), and a
    second replay is timed between two events on the launch stream.
    """
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def flush():
        for j in range(max(0, copies - steps)):
            step(first + steps + j, launches)

    if use_graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(steps):
                    step(first + i, launches)
        torch.cuda.synchronize()
        g.replay()
        flush()
        torch.cuda.synchronize()
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b), "graph replay"
    flush()
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        step(first + i, launches)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b), "eager launches"


# ---------------------------------------------------------------------------
# workloads: each returns (step(i, launches), info) with device data prepared
# ---------------------------------------------------------------------------

MAX_COPIES = 64


def _copies(total_bytes):
    # tiny layers (the 256x256 case) cannot defeat the caches with a sane number of copies:
    # they are latency-bound and their number is reported as such
    return max(1, min(MAX_COPIES, math.ceil(CACHE_DEFEAT_BYTES / total_bytes)))


# The decoder layer's launch groups when layers that read one input vector are fused:
# q/k/v read the attention input, gate/up the MLP input (each group one launch).
FUSED_GROUPS = {3: [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")), ("down", ("down",))]}
FUSED = {"on": True}
# --int8: batch-1 layers carry TG_FLAG_INT8_ACT (mul1 with the int8 form of x~)
LAYER_FLAGS = {"int8": False}


def batch1_flags(tg):
    return tg.TG_FLAG_INT8_ACT if LAYER_FLAGS["int8"] else 0


def launch_groups(workload, names):
    """[(launch name, tensor names)]: one launch per tensor, or the fused groups."""
    if FUSED["on"] and workload in FUSED_GROUPS:
        return FUSED_GROUPS[workload]
    return [(n, (n,)) for n in names]


def group_inputs(inputs, wl, members, code_id, copy=0):
    """{tensor: (layer arrays, x bits)} of one launch group's tensors in one copy: every layer of a
    fused group reads the input vector of the group's first tensor."""
    names = list(wl.tensors)
    x = inputs.make_x(wl.tensors[members[0]][1], wl.seed, tensor=names.index(members[0]), copy=copy)
    out = {}
    for name in members:
        m, n, k = wl.tensors[name]
        out[name] = (inputs.make_layer(m, n, k, wl.seed, tensor=names.index(name), copy=copy, code_id=code_id), x)
    return out


def linear_inputs(inputs, wl, workload, code_id, copy=0):
    """{tensor: (layer arrays, x bits)} of one copy of the whole workload, as the bench's launches read them."""
    out = {}
    for _, members in launch_groups(workload, list(wl.tensors)):
        out.update(group_inputs(inputs, wl, members, code_id, copy))
    return out


def setup_linears(torch, tg, inputs, wl, dev, code_id, workload=3):
    """Workloads 1-3: batch-1 GEMVs over the workload's tensors, each launch group once per step.
    Every launch group has its own number of seeded copies (>= 1 GiB of codes each, at most 64), so
    a launch never reads a copy it read less than 1 GiB of its own launches ago."""
    names = list(wl.tensors)
    groups = launch_groups(workload, names)
    code_bytes = sum(m * n * k // 8 for (m, n, k) in wl.tensors.values())
    gbytes = {g: sum(wl.tensors[t][0] * wl.tensors[t][1] * wl.tensors[t][2] // 8 for t in members)
              for g, members in groups}
    copies = {g: _copies(b) for g, b in gbytes.items()}
    log(f"{wl.name}: {len(names)} tensor(s) in {len(groups)} launch(es), {code_bytes} code bytes per step, "
        f"copies per launch {copies}")
    per = {g: [] for g, _ in groups}
    for g, members in groups:
        for c in range(copies[g]):
            arrays = group_inputs(inputs, wl, members, code_id, copy=c)
            Ls = [tg.DeviceLayer(arrays[t][0], dev, flags=batch1_flags(tg)) for t in members]
            x = tg.fp16_tensor(arrays[members[0]][1], dev)
            ys = [torch.empty(L.m, dtype=torch.float32, device=dev) for L in Ls]
            per[g].append((Ls, x, ys))
    ws = {g: (tg.fused_workspace(per[g][0][0], dev) if len(members) > 1 else tg.workspace(per[g][0][0][0], 1, dev))
          for g, members in groups}

    def step(i, launch):
        s = torch.cuda.current_stream()
        for g, members in groups:
            Ls, x, ys = per[g][i % copies[g]]
            if len(members) > 1:
                launch(g, lambda Ls=Ls, x=x, ys=ys, w=ws[g]: tg.trellis_gemv_fused(Ls, x, ys, w, s))
            else:
                launch(g, lambda L=Ls[0], x=x, y=ys[0], w=ws[g]: tg.trellis_gemv(L, x, y, w, s))

    alg = {g: sum(gemv_bytes(*wl.tensors[t]) - (2 * wl.tensors[t][1] if j else 0) for j, t in enumerate(members))
           for g, members in groups}
    fused = any(len(m) > 1 for _, m in groups)
    units = "layer" if len(names) == 1 else \
        f"decoder layer (7 GEMVs in {len(groups)} launches{', q/k/v and gate/up fused' if fused else ''})"
    return step, dict(code_bytes=code_bytes, copies=max(copies.values()), copies_per_launch=copies, alg_bytes=alg,
                      names=[g for g, _ in groups], mfma=False, units=units, k_bits={g: wl.tensors[m[0]][2]
                                                                                     for g, m in groups},
                      weights={g: sum(wl.tensors[t][0] * wl.tensors[t][1] for t in members) for g, members in groups})


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




def run_gpu(workload, steps, warmup, use_graph, code_id=0, hot=True):
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
    if workload in (1, 2, 3):
        step, info = setup_linears(torch, tg, inputs, wl, dev, code_id, workload)
    else:
        setup = {4: setup_gemm, 5: setup_moe, 6: setup_prefill, 7: setup_moe_block}[workload]
        step, info = setup(torch, tg, inputs, wl, dev, code_id)
    dom = max(info["names"], key=lambda k: info["alg_bytes"][k])     # kernel moving the most bytes
    copies = info["copies"]
    for i in range(warmup):
        step(i, Launches())
    torch.cuda.synchronize()
    eager_ms, _ = timed_steps_ms(torch, step, warmup, steps, copies, Launches(), False)
    region_ms, timing = eager_ms, "eager launches"
    dom_ms = None
    if use_graph:
        try:
            region_ms, timing = timed_steps_ms(torch, step, warmup, steps, copies, Launches(), True)
            dom_ms, _ = timed_steps_ms(torch, step, warmup, steps, copies, Launches(only=dom), True)
        except Exception as e:  # noqa: BLE001 - keep the eager number
            log("graph replay unavailable:", repr(e))
    if dom_ms is None:
        dom_ms, _ = timed_steps_ms(torch, step, warmup, steps, copies, Launches(only=dom), False)
    # Context only, never the metric: the same copy every step (its code words stay in the caches).
    hot_ms = None
    if hot and timing == "graph replay":
        hot_ms, _ = timed_steps_ms(torch, lambda i, launches: step(0, launches), 0, steps, 1, Launches(), True)
    return info, dict(region_ms=region_ms, eager_ms=eager_ms, dom=dom, dom_ms=dom_ms, timing=timing, hot_ms=hot_ms)


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


def decode_ceiling(k_bits, code_id, flags=0):
    """Decoded weights per second of the decode-only probe (the batch-1 loop on LDS-resident code words):
    the best of 256, 512 and 1024 workgroups of 8 waves (2, 4 and 8 waves per SIMD)."""
    import torch
    from trellis_coded_gemv_amd import binding as tg
    steps = 256
    best = None
    for wgs in (256, 512, 1024):
        out = torch.empty(wgs * 512, dtype=torch.float32, device="cuda")
        tg.decode_ceiling(k_bits, code_id, wgs, steps, out, flags=flags)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            tg.decode_ceiling(k_bits, code_id, wgs, steps, out, flags=flags)
        b.record()
        torch.cuda.synchronize()
        rate = 5 * wgs * 512 * 64 * steps / (a.elapsed_time(b) * 1e-3)
        best = rate if best is None or rate > best else best
    return best


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


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, untuned, on a bounded sample of the workload, on every core of the
# process's affinity mask (one worker process per core, forked before the GPU is touched).
# ---------------------------------------------------------------------------

_CPU_JOB = {}


def _cpu_item(item):
    """One unit of oracle work: (kind, key, ...). Returns (code bytes, oracle output)."""
    from oracle import gemv as ogemv
    kind = item[0]
    if kind == "block":                      # one 128-output block of a tensor, all its activation rows
        _, name, b = item
        arr, X = _CPU_JOB["layers"][name]
        rows = np.arange(128 * b, 128 * b + 128)
        if _CPU_JOB.get("int8"):
            y = ogemv.gemv_int8_rows(arr, X, rows)
        else:
            y = ogemv.gemv_rows(arr, X, rows) if X.ndim == 1 else ogemv.gemm_rows(arr, X, rows)
        return 128 * arr.n * arr.k_bits // 8, y
    if kind == "token":                      # a whole MoE block (workload 7) or its 24 GEMVs (workload 5)
        from oracle import moe
        _, t = item
        gu, dn, sel, w, x, xd = _CPU_JOB["tokens"][t]
        nbytes = sum(a.code_bytes for a in list(gu.values()) + list(dn.values()))
        if _CPU_JOB["block"]:
            return nbytes, moe.moe_block(gu, dn, sel, w, x)
        ys = [ogemv.gemv(gu[2 * int(e) + k], x) for e in sel for k in (0, 1)]
        ys += [ogemv.gemv(dn[int(e)], xd[i]) for i, e in enumerate(sel)]
        return nbytes, ys[0]
    raise ValueError(kind)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(workload, code_id=0, blocks_per_tensor=32, tokens=16, max_workers=16):
    """Time the oracle on a sample of the workload with one process per core of the affinity mask
    (at most max_workers). Returns (baseline record, oracle outputs for the parity spot check)."""
    import multiprocessing as mp
    from trellis_coded_gemv_amd import inputs

    wl = workload_of(inputs, workload)
    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(affinity, max_workers))
    _CPU_JOB.clear()
    if workload in (5, 7):
        _CPU_JOB["block"] = workload == 7
        _CPU_JOB["tokens"] = {}
        for t in range(min(tokens, wl.tokens)):
            gu, dn, sel, w, x = _moe_token(inputs, wl, code_id, t)
            xd = inputs.make_x(wl.inter, wl.seed, tensor=20_000 + t, rows=wl.top_k)
            _CPU_JOB["tokens"][t] = (gu, dn, sel, w, x, xd)
        items = [("token", t) for t in _CPU_JOB["tokens"]]
        what = f"{len(items)} tokens, {'the whole block' if workload == 7 else 'their 24 expert GEMVs'} each"
        scale = 1.0
    else:
        _CPU_JOB["layers"] = {}
        _CPU_JOB["int8"] = LAYER_FLAGS["int8"] and wl.batch == 1
        items = []
        Mo = min(wl.batch, 16)               # oracle rows per block; the rate is scaled to the step's rows
        arrays = linear_inputs(inputs, wl, workload, code_id) if wl.batch == 1 else None
        for ti, (name, (m, n, k)) in enumerate(wl.tensors.items()):
            if arrays is not None:           # the batch-1 step's own inputs (shared within a fused group)
                arr, X = arrays[name]
            else:
                arr = inputs.make_layer(m, n, k, wl.seed, tensor=ti, code_id=code_id)
                X = inputs.make_x(n, wl.seed, tensor=ti, rows=Mo)
            _CPU_JOB["layers"][name] = (arr, X)
            nb = m // 128
            blocks = np.unique(np.linspace(0, nb - 1, min(blocks_per_tensor, nb)).astype(int))
            items += [("block", name, int(b)) for b in blocks]
        what = (f"{len(items)} 128-output blocks over the tensors {', '.join(wl.tensors)}"
                f" (decode + fp64 GEMV{'' if Mo == 1 else f' of {Mo} rows, scaled to {wl.batch}'}"
                f"{', int8 form of x~' if _CPU_JOB['int8'] else ''})")
        scale = wl.batch / Mo
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        pool.map(_cpu_item, items[:workers], chunksize=1)     # warm-up: workers started, code paged in
        t0 = time.perf_counter()
        res = pool.map(_cpu_item, items, chunksize=1)
        dt = time.perf_counter() - t0
    nbytes = sum(r[0] for r in res)
    rate = nbytes / (dt * scale)
    rec = {"value": round(rate / 1e9, 6), "unit": "GB/s", "cores": workers, "kind": "oracle",
           "sample": f"{what}: {nbytes} code bytes in {dt:.1f} s wall on {workers} worker processes",
           "affinity_cores": affinity, "cpu_count": os.cpu_count(), "cpu_model": _cpu_model()}
    refs = {item: r[1] for item, r in zip(items, res)}
    _CPU_JOB.clear()
    return rec, refs


def parity_spot_check(workload, code_id, refs):
    """Copy 0 of the workload on the GPU against the oracle outputs the CPU baseline computed
    (a few of its sampled blocks or tokens); max |dy| / max |y_ref| over them."""
    import torch
    from trellis_coded_gemv_amd import binding as tg
    from trellis_coded_gemv_amd import inputs

    wl = workload_of(inputs, workload)
    errs = []
    if workload in (5, 7):
        t = 0
        ref = refs[("token", t)]
        gu, dn, sel, w, x = _moe_token(inputs, wl, code_id, t)
        if workload == 7:
            gut = tg.LayerTable([tg.DeviceLayer(wl.layer(e, k, code_id=code_id), "cuda") for e in range(wl.experts)
                                 for k in ("gate", "up")], "cuda")
            dnt = tg.LayerTable([tg.DeviceLayer(wl.layer(e, "down", code_id=code_id), "cuda")
                                 for e in range(wl.experts)], "cuda")
            y = tg.trellis_moe_block(gut, dnt, torch.from_numpy(sel).to("cuda"), torch.from_numpy(w).to("cuda"),
                                     tg.fp16_tensor(x, "cuda"))
        else:
            y = tg.trellis_gemv(tg.DeviceLayer(gu[2 * int(sel[0])], "cuda"), tg.fp16_tensor(x, "cuda"))
        torch.cuda.synchronize()
        return float(np.abs(y.cpu().numpy() - ref).max() / np.abs(ref).max())
    by_tensor = {}
    for item, y in refs.items():
        by_tensor.setdefault(item[1], []).append((item[2], y))
    if wl.batch == 1:                        # the step's own launches on copy 0
        arrays = linear_inputs(inputs, wl, workload, code_id)
        for _, members in launch_groups(workload, list(wl.tensors)):
            Ls = [tg.DeviceLayer(arrays[t][0], "cuda", flags=batch1_flags(tg)) for t in members]
            x = tg.fp16_tensor(arrays[members[0]][1], "cuda")
            ys = tg.trellis_gemv_fused(Ls, x) if len(members) > 1 else [tg.trellis_gemv(Ls[0], x)]
            torch.cuda.synchronize()
            for name, y in zip(members, ys):
                y = y.cpu().numpy()
                for b, ref in by_tensor.get(name, []):
                    errs.append(float(np.abs(y[128 * b:128 * b + 128] - ref).max() / np.abs(ref).max()))
        return max(errs) if errs else None
    for ti, (name, (m, n, k)) in enumerate(wl.tensors.items()):
        arr = inputs.make_layer(m, n, k, wl.seed, tensor=ti, code_id=code_id)
        Mo = min(wl.batch, 16)
        X = inputs.make_x(n, wl.seed, tensor=ti, rows=Mo)
        L = tg.DeviceLayer(arr, "cuda")
        if workload == 6:
            Y = tg.trellis_gemm_prefill(L, tg.fp16_tensor(X, "cuda"))
        else:
            Y = tg.trellis_gemm_small(L, tg.fp16_tensor(X, "cuda"))
        torch.cuda.synchronize()
        Y = Y.cpu().numpy()
        for b, ref in by_tensor.get(name, []):
            ref = np.atleast_2d(ref)
            got = Y[:, 128 * b:128 * b + 128]
            errs.append(float(np.abs(got - ref).max() / np.abs(ref).max()))
    return max(errs) if errs else None


def measure(workload, code_id, steps, warmup, use_graph, hot=True):
    """One workload's timing record (no CPU baseline)."""
    from trellis_coded_gemv_amd import inputs
    wl = workload_of(inputs, workload)
    info, t = run_gpu(workload, steps, warmup, use_graph, code_id, hot)
    ms_per_step = t["region_ms"] / steps
    value = info["code_bytes"] / (ms_per_step * 1e-3) / 1e9
    dom = t["dom"]
    dom_launch_ms = t["dom_ms"] / steps
    rec = {"workload": wl.name + ("_block" if workload == 7 else ""), "code_id": code_id,
           "int8_activations": bool(LAYER_FLAGS["int8"] and workload in (1, 2, 3)), "units": info["units"],
           "us_per_step": round(ms_per_step * 1e3, 3), "gbs": round(value, 2),
           "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2), "timing": t["timing"],
           "dominant": dom, "dominant_launch_us": round(dom_launch_ms * 1e3, 3)}
    if "flops" in info:
        tf = info["flops"] / (dom_launch_ms * 1e-3) / 1e12
        rec["mfma_tflops"] = round(tf, 2)
        rec["mfma_frac_of_dense_f16_peak"] = round(tf / MFMA_F16_PEAK_TFLOPS, 5)
    return info, t, rec, value, ms_per_step, dom_launch_ms


def context_codes(text, code_id, int8, workload):
    """The (code_id, int8) pairs of a --context-codes list ('3,2i8,1'), without the line's own and
    without int8 forms the workload cannot run (mul1's int8 form, batch-1 workloads only)."""
    out = []
    for spec in [v.strip() for v in text.split(",") if v.strip()]:
        i8 = spec.endswith("i8")
        cid = int(spec[:-2] if i8 else spec)
        if cid not in (0, 1, 2, 3):
            raise ValueError(f"unknown code in --context-codes: {spec}")
        if (cid, i8) == (code_id, int8) or (i8 and (cid != 2 or workload not in (1, 2, 3))):
            continue
        out.append((cid, i8))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=[1, 2, 3, 4, 5, 6, 7])
    ap.add_argument("--code", type=int, default=0, choices=[0, 1, 2, 3],
                    help="code_id of every layer: 0 the three-instruction code, 1 the pair code, 2 mul1, 3 MCG")
    ap.add_argument("--int8", action="store_true",
                    help="with --code 2: the batch-1 layers multiply by the int8 form of x~ (TG_FLAG_INT8_ACT)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="workload 3: one launch per tensor (default: q/k/v and gate/up in one launch each)")
    ap.add_argument("--cpu-blocks", type=int, default=32,
                    help="oracle sample: 128-output blocks per tensor (tokens for workloads 5/7); 0 skips it")
    ap.add_argument("--context", default="2,4,5",
                    help="comma-separated workloads also measured briefly as context ('' for none)")
    ap.add_argument("--context-codes", default="3,2i8,1",
                    help="comma-separated codes (a trailing 'i8': mul1 with int8 activations) also measured "
                         "briefly on the bench's workload as context ('' for none)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="after timing, write (fill) and read (sum) this many MiB (counter calibration)")
    args = ap.parse_args(argv)
    FUSED["on"] = not args.unfused
    if args.int8 and args.code != 2:
        print("--int8 needs --code 2 (the int8 form is mul1's)", file=sys.stderr)
        return 2
    LAYER_FLAGS["int8"] = args.int8
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library has no multi-GPU path.",
              file=sys.stderr)
        return 2

    # the CPU baseline runs first: its worker processes are forked before anything touches the GPU
    cpu, refs = (None, None)
    if args.cpu_blocks > 0:
        log("cpu baseline (oracle) ...")
        cpu, refs = cpu_baseline(args.workload, args.code, blocks_per_tensor=args.cpu_blocks,
                                 tokens=min(args.cpu_blocks, 16))
        log("cpu baseline:", cpu["value"], "GB/s on", cpu["cores"], "workers")

    import torch
    from trellis_coded_gemv_amd import binding as tg
    from trellis_coded_gemv_amd import inputs
    wl = workload_of(inputs, args.workload)
    steps = args.steps
    info, t, rec, value, ms_per_step, dom_launch_ms = measure(args.workload, args.code, steps, args.warmup,
                                                              not args.no_graph)
    dom = t["dom"]
    achieved = info["alg_bytes"][dom] / (dom_launch_ms * 1e-3) / 1e9
    config = {"workload": rec["workload"], "units": info["units"], "code_bytes_per_step": int(info["code_bytes"]),
              "copies": info.get("copies_per_launch", info["copies"]), "us_per_step": rec["us_per_step"],
              "pct_of_hbm_peak": rec["pct_of_hbm_peak"], "timing": t["timing"],
              "eager_us_per_step": round(t["eager_ms"] / steps * 1e3, 3),
              "code_id": args.code, "int8_activations": rec["int8_activations"], "build_id": tg.build_id()}
    if args.workload not in (5, 7):
        config.update({"tensors": {k: list(v) for k, v in wl.tensors.items()}, "batch": wl.batch})
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(args.workload, dom, args.code),
            "algorithmic_bytes": int(info["alg_bytes"][dom]), "launch_us": round(dom_launch_ms * 1e3, 3)}
    if not info["mfma"]:
        k_dom = info["k_bits"][dom] if "k_bits" in info else 2
        cflags = tg.TG_FLAG_INT8_ACT if rec["int8_activations"] else 0
        ceil = decode_ceiling(k_dom, args.code, cflags)
        wps = info["weights"][dom] / (dom_launch_ms * 1e-3)
        roof["alu"] = {"achieved": round(wps / 1e9, 2), "ceiling": round(ceil / 1e9, 2), "unit": "G weights/s",
                       "frac": round(wps / ceil, 4), "ceiling_kernel": f"tg_decode_ceiling(k_bits={k_dom}, "
                                                                    f"code_id={args.code}, flags={cflags})"}
    if "flops" in info:
        tf = info["flops"] / (dom_launch_ms * 1e-3) / 1e12
        roof["mfma"] = {"achieved": round(tf, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 5)}
    if info.get("prefill"):
        # the contraction on the matrix cores is the roofline here
        mf = roof.pop("mfma")
        hbm = {k: roof.pop(k) for k in ("achieved", "peak", "unit", "frac", "algorithmic_bytes")}
        roof.update({"bound": "mfma", "achieved": mf["achieved"], "peak": mf["peak"], "unit": "TFLOP/s",
                     "frac": mf["frac"], "algorithmic_flops": info["flops"], "hbm": hbm})
    config["context"] = {
        "hot_cache_us_per_step": None if t["hot_ms"] is None else round(t["hot_ms"] / steps * 1e3, 3),
        "stream_read_gbs": stream_read_gbs(torch),
        "note": "hot: copy 0 every step (caches warm); stream_read: torch.sum over 1 GiB (fp64 view)"}
    if refs is not None:
        config["parity_max_rel_err"] = parity_spot_check(args.workload, args.code, refs)
    others = []
    for w in [int(v) for v in args.context.split(",") if v.strip()]:
        if w == args.workload:
            continue
        log("context workload", w)
        _, _, r, _, _, _ = measure(w, args.code, steps, args.warmup, not args.no_graph, hot=False)
        others.append(r)
    config["other_workloads"] = others
    codes = []
    for cid, i8 in context_codes(args.context_codes, args.code, args.int8, args.workload):
        log("context code", cid, "int8" if i8 else "")
        saved = LAYER_FLAGS["int8"]
        LAYER_FLAGS["int8"] = i8
        try:
            _, _, r, _, _, _ = measure(args.workload, cid, steps, args.warmup, not args.no_graph, hot=False)
        finally:
            LAYER_FLAGS["int8"] = saved
        codes.append(r)
    config["other_codes"] = codes
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8" if rec["int8_activations"] else "fp16", "data": "synthetic",
        "config": config, "roofline": roof,
    }
    if args.copy_calib_mb > 0:
        # counter calibration: a pure write (fill) and a pure read (sum) of known size
        buf = torch.empty(args.copy_calib_mb << 18, dtype=torch.float32, device="cuda")
        for _ in range(3):
            buf.fill_(1.0)
            buf.sum()
        torch.cuda.synchronize()
        out["config"]["calibration_bytes"] = buf.numel() * 4
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

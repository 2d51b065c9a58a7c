#!/usr/bin/env python3
"""Benchmark of the FastMKA layer forward on one MI355X (gfx950).

One step = one whole-layer prefill of the Llama-3.1-8B-shaped layer (batch 1,
65536 tokens, D=4096, 32 query / 8 KV heads of 128, bf16) through the
composite C-ABI call mka_prefill: route (Q projection + router), EMA scan and
block means, block index and projections, retrieval, fusion + K/V
projection, causal flash attention.  Inputs are resident in HBM before timing
starts.  ``value`` is prefill tokens/s.  Before the warmup, untimed
back-to-back steps run for ``--settle-ms`` (the GPU's clocks ramp up over tens
of milliseconds of load after an idle spell).  A second loop issues the stage
calls one by one with HIP events between them for the per-stage breakdown and
the attention roofline.

The same line carries the Qwen2.5-7B-shaped prefill workloads (2 x 4096 and
1 x 32768 tokens) with the same figures, the decode measurement (the
131072-token fused cache workload, 256 decode steps of ``mka_decode_step``:
median microseconds per token, with three layers' caches taken in turn so
that every step reads its cache from HBM, and with one layer re-read for
comparison), and the CPU oracle timed on bounded samples.

Also by default (``--quick`` skips them): a training step (forward and
backward), the paged cache, batched decode, full MKA and the routing variants
on the 2 x 4096 workload, each as its own object of the line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FastMKA layer prefill tokens/s + decode µs/tok at 1 GPU; % MFMA / HBM peak"
PEAK_BF16_FLOPS = 2.5e15  # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12   # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Hardware-counter traffic (rocprofv3 FETCH_SIZE / WRITE_SIZE, KiB per dispatch)
# is taken in two profiled runs of this script and summarised into a JSON file
# per workload under profiles/; the counters are scaled by what they read for a
# plain copy kernel of known size.  Each kernel's entry records a hash of the
# sources it is built from, and a figure is reported only while that hash
# still matches.
CSRC = os.path.join(ROOT, "route_kv_memory_amd", "csrc")
KERNEL_SOURCES = {
    "attn_prefill_bf16_kernel": ["attn.hip"],
    "attn_decode_split_kernel": ["attn.hip", "attn_split.h"],
    "decode_attend_kernel": ["decode.hip", "attn_split.h"],
    "decode_inputs_kernel": ["decode.hip"],
    "mka::decode_merge_kernel": ["decode.hip", "attn_split.h"],
    "attn_decode_merge_kernel": ["attn.hip", "attn_split.h"],
    "mka::EpiStore<unsigned short>": ["gemm.hip", "gemm.h"],  # Q projection (bf16 GEMM)
    "mka::EpiKV<unsigned short>": ["gemm.hip", "gemm.h"],     # fused K/V projection
    "ema_pass1": ["ema.hip"],
    "ema_pass2": ["ema.hip"],
    "ema_pass3": ["ema.hip"],
    "router_mfma_kernel": ["route.hip"],
    "simhash_split_kernel": ["l3.hip"],
    "fuse_mix_kernel": ["fuse.hip"],
    "fuse_mix_sel_kernel": ["fuse.hip"],
    "fuse_split_kernel": ["fuse.hip"],
    "topr_rows_kernel": ["l3.hip"],
}
ROOFLINE_KERNEL = "attn_prefill_bf16_kernel"


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


# The abstract page's ablations: Table 10 (fixed lambda = 1/3, hard top-2,
# hard top-1) and Table 9 (L1+L2, L1+L3, L1 alone), as (route_mode, tiers).
VARIANTS = [("fixed", "l1l2l3"), ("top2", "l1l2l3"), ("top1", "l1l2l3"), ("soft", "l1l2"),
            ("soft", "l1l3"), ("soft", "l1")]
COPY_KERNEL = "neg_kernel"  # torch.neg(out=): one read and one write per element


def source_hash(kernel):
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["common.h", "kernels.h"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    from route_kv_memory_amd.build import HIPCC_FLAGS

    h.update(" ".join(HIPCC_FLAGS[:-2]).encode())  # flags, without the include path
    return h.hexdigest()[:16]


def copy_calibration(mib):
    """A plain copy of ``mib`` MiB (fp32 in, fp32 out), three launches."""
    import torch

    n = mib * 2**20 // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def traffic_summary(fetch_csv, write_csv, copy_mib, commands):
    """Per-dispatch HBM bytes of the kernels in KERNEL_SOURCES from two
    rocprofv3 --pmc runs, each counter scaled by its copy-kernel reading."""
    import csv
    import collections

    def per_kernel(path, counter):
        acc = collections.defaultdict(list)
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return acc

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")

    def mean_of(acc, sub):
        vals = [v for k, vs in acc.items() if sub in k for v in vs]
        if not vals:
            raise SystemExit(f"no dispatch of {sub} in the counter file; kernels: {sorted(acc)[:8]}")
        return float(np.mean(vals)), len(vals)

    copy_kib = copy_mib * 1024.0
    cf, _ = mean_of(fetch, COPY_KERNEL)
    cw, _ = mean_of(write, COPY_KERNEL)
    out = {"commands": commands, "copy_kernel": f"torch.neg, {copy_mib} MiB in and out",
           "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": copy_kib / cf, "write_scale": copy_kib / cw, "kernels": {}}
    for k in KERNEL_SOURCES:
        try:
            fk, nf = mean_of(fetch, k)
            wk, nw = mean_of(write, k)
        except SystemExit:
            continue
        byt = (fk * out["fetch_scale"] + wk * out["write_scale"]) * 1024.0
        out["kernels"][k] = {"fetch_kib": fk, "write_kib": wk, "dispatches": [nf, nw],
                             "bytes_per_launch": byt, "source_hash": source_hash(k)}
    return out


def traffic_for(kernel, workload):
    """Calibrated HBM bytes per launch of ``kernel`` on ``workload``, or None
    when no counters were taken for the current source of that kernel."""
    try:
        with open(traffic_file(workload)) as fh:
            entry = json.load(fh)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    return entry["bytes_per_launch"] if entry["source_hash"] == source_hash(kernel) else None


def prefill_flops(s):
    M = s.batch * s.seq
    qw, kvw, D = s.q_width, s.kv_width, s.d_model
    pairs = s.batch * s.n_heads * s.seq * (s.seq + 1) // 2
    return {
        "route": 2.0 * M * qw * D + 2.0 * M * qw * s.router_hidden,
        "fuse_kv": 2.0 * M * 2 * kvw * D,
        "attn": 4.0 * s.head_dim * pairs,
    }


def settle(step_fn, ms):
    """Untimed back-to-back steps for ``ms`` milliseconds of wall time: after an
    idle spell the GPU's clocks take tens of milliseconds of load to come back
    up, which a few warmup steps do not cover.  Returns the steps run."""
    import torch

    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step_fn()
        n += 8
        torch.cuda.synchronize()
    return n


def bench_prefill(s, steps, warmup, variants=(), settle_ms=0.0, full=False):
    import torch

    from route_kv_memory_amd import mka
    from route_kv_memory_amd.inputs import prefill_inputs
    from route_kv_memory_amd.layer import Layer, to_device

    log(f"prefill: generating {s.name} inputs")
    inp = prefill_inputs(s)
    N = s.seq
    layer = Layer(s, inp, t_cap=N, nb_cap=N // s.block, full=full)
    x = to_device(inp["x"], s.dtype)
    del inp
    out = layer.outputs(N)
    d = layer.dims(N)
    ws = layer.workspace(mka.mka_workspace_bytes(d, mka.MKA_OP_PREFILL))
    nws = ws.numel()
    st, w = layer.st, layer.w
    stream = torch.cuda.current_stream()
    names = ["route", "ema", "index", "retrieve", "fuse_kv", "attn"]
    nb = N // s.block

    def step(ev):
        ev[0].record(stream)
        mka.mka_route(d, x, w["w_q"], w["w_r1"], w["w_r2"], out["q"], out["lambda"], ws, nws,
                      stream)
        ev[1].record(stream)
        mka.mka_ema_scan(d, x, 0, st["ema_state"], st["block_acc"], out["l2"], st["block_means"],
                         layer.nb_cap, ws, nws, stream)
        ev[2].record(stream)
        mka.mka_l3_index(d, st["block_means"], layer.nb_cap, 0, nb, w["proj"], st["block_hash"],
                         ws, nws, stream)
        mka.mka_l3_block_kv(d, st["block_means"], layer.nb_cap, 0, nb, w["w_k"], w["w_v"],
                            st["block_kv"], stream)
        ev[3].record(stream)
        mka.mka_l3_retrieve(d, out["l2"], w["proj"], st["block_hash"], layer.nb_cap, 0, out["key"],
                            out["idx"], ws, nws, stream)
        ev[4].record(stream)
        mka.mka_fuse_kv_proj(d, x, out["l2"], st["block_means"], layer.nb_cap, out["idx"],
                             out["lambda"], w["w_k"], w["w_v"], st["k_cache"], st["v_cache"], 0,
                             layer.t_cap, ws, nws, stream)
        ev[5].record(stream)
        mka.mka_attn_prefill(d, out["q"], st["k_cache"], st["v_cache"], layer.t_cap, 0, out["o"],
                             stream)
        ev[6].record(stream)

    # Timed: the composite mka_prefill (the summary chain on the library's
    # auxiliary stream beside the query product).  Every step starts from an
    # empty prefix (pos0 = 0), for which the state buffers are not read.
    settled = settle(lambda: layer.prefill(x, 0, out=out, stream=stream), settle_ms)

    def composite(fn=layer.prefill):
        ev_step = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for _ in range(warmup):
            fn(x, 0, out=out, stream=stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            ev_step[k][0].record(stream)
            fn(x, 0, out=out, stream=stream)
            ev_step[k][1].record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        return wall * 1e3, float(np.mean([e[0].elapsed_time(e[1]) for e in ev_step]))

    wall_ms, gpu_ms = composite()
    # Routing variants: the same buffers and inputs, the layer's shape swapped.
    var_ms = {}
    for mode, tiers in variants:
        layer.shape = s.replace(route_mode=mode, tiers=tiers)
        var_ms[f"{mode}/{tiers}"] = composite()[0]
        log(f"prefill variant {mode}/{tiers}: {var_ms[f'{mode}/{tiers}']:.4f} ms")
    layer.shape = s
    # Full MKA (three attention paths) on the same inputs.
    full_ms = composite(layer.full_prefill)[0] if full else None
    if full:
        log(f"prefill full MKA: {full_ms:.4f} ms")

    # Breakdown: the same calls one by one on one stream, HIP events between
    # them (the attention stage is exactly one kernel launch).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    step(evs[0])
    torch.cuda.synchronize()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
                for i, n in enumerate(names)}
    seq_ms = float(np.mean([e[0].elapsed_time(e[6]) for e in evs]))
    return dict(wall_ms=wall_ms, gpu_ms=gpu_ms, stage_ms=stage_ms, sequential_ms=seq_ms,
                variants_ms=var_ms, settle_steps=settled, full_ms=full_ms)


def bench_train(s, steps, warmup, settle_ms=0.0):
    """One training step of the layer: mka_prefill (which saves each query row's
    log-sum-exp) then mka_backward with a seeded dO; HIP events split the two."""
    import torch

    from route_kv_memory_amd.inputs import prefill_inputs, round_bf16
    from route_kv_memory_amd.layer import Layer, to_device

    inp = prefill_inputs(s)
    layer = Layer(s, inp, t_cap=s.seq, nb_cap=s.seq // s.block)
    x = to_device(inp["x"], s.dtype)
    del inp
    d_o = to_device(round_bf16(np.random.default_rng(s.seed + 1000).standard_normal(
        (s.batch, s.seq, s.n_heads, s.head_dim))), s.dtype)
    out, grads = layer.outputs(s.seq), layer.grads(s.seq)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        layer.prefill(x, 0, out=out, stream=stream)
        if ev:
            ev[1].record(stream)
        layer.backward(x, out, d_o, grads, stream=stream)
        if ev:
            ev[2].record(stream)

    settle(step, settle_ms)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    # the attention backward alone (mka_attn_backward), for its roofline
    from route_kv_memory_amd import mka

    d = layer.dims(s.seq)
    dq = torch.empty(s.batch, s.seq, s.n_heads, s.head_dim, device="cuda")
    dkv = torch.empty(s.batch, s.seq, 2, s.n_kv_heads, s.head_dim, device="cuda")
    ws = torch.empty(max(256, mka.mka_workspace_bytes(d, mka.MKA_OP_ATTN_BACKWARD)),
                     dtype=torch.uint8, device="cuda")

    def attn_bwd():
        mka.mka_attn_backward(d, out["q"], layer.st["k_cache"], layer.st["v_cache"], layer.t_cap,
                              out["o"], out["lse"], d_o, dq, dkv, ws, ws.numel(), stream)

    attn_bwd()
    a_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    a_ev[0].record(stream)
    for _ in range(steps):
        attn_bwd()
    a_ev[1].record(stream)
    torch.cuda.synchronize()
    return dict(ms=wall, fwd_ms=float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
                bwd_ms=float(np.mean([e[1].elapsed_time(e[2]) for e in evs])),
                attn_bwd_ms=a_ev[0].elapsed_time(a_ev[1]) / steps)


def bench_prefill_paged(s, steps, warmup, page_size, settle_ms=0.0):
    """The composite prefill with a paged fused cache (pages of ``page_size``
    rows, a seeded random order with spare pages in the pool)."""
    import torch

    from route_kv_memory_amd.inputs import prefill_inputs
    from route_kv_memory_amd.layer import Layer, to_device

    inp = prefill_inputs(s)
    layer = Layer(s, inp, t_cap=s.seq, nb_cap=s.seq // s.block, page_size=page_size,
                  spare_pages=8)
    x = to_device(inp["x"], s.dtype)
    del inp
    out = layer.outputs(s.seq)
    stream = torch.cuda.current_stream()
    settle(lambda: layer.prefill(x, 0, out=out, stream=stream), settle_ms)
    for _ in range(warmup):
        layer.prefill(x, 0, out=out, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.prefill(x, 0, out=out, stream=stream)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def bench_decode(s, steps, warmup, variants=(), full=False, page_size=None, copies=1):
    """Decode steps of the workload ``s``.  ``copies`` > 1: that many layers
    (weights, state and fused cache each), taken in turn step by step, so that
    a step's cache and weights were last read ``copies - 1`` steps earlier;
    with three copies (about 0.9 GB) every step reads them from HBM rather than
    from the 256 MB last-level cache.  Routing variants and full MKA run on the
    first copy alone."""
    import torch

    from route_kv_memory_amd import mka
    from route_kv_memory_amd.inputs import decode_inputs
    from route_kv_memory_amd.layer import Layer, to_device

    log(f"decode: generating {s.name} state ({copies} cop{'y' if copies == 1 else 'ies'})")
    dec = decode_inputs(s)
    T0, n = s.decode_cached, s.decode_steps
    t_cap = T0 + n
    nb0 = T0 // s.block
    layers = []
    for i in range(copies):
        lay = Layer(s, dec, t_cap=t_cap, nb_cap=t_cap // s.block + 1, full=full and i == 0,
                    page_size=page_size, spare_pages=8 if page_size else 0)
        lay.load_cache("k", to_device(dec["k_cache"], s.dtype))
        lay.load_cache("v", to_device(dec["v_cache"], s.dtype))
        layers.append(lay)
    layer = layers[0]
    st = layer.st
    if full:  # the three tiers' caches hold the same synthetic rows (timing only)
        for c in ("k", "v"):
            for t in layer.kv3[c]:
                t[:, :, :T0].copy_(st[f"{c}_cache"][:, :, :T0])
    init = {k: to_device(dec[k]) for k in ("ema_state", "block_acc")}
    means0 = to_device(dec["block_means"])
    tokens = to_device(dec["tokens"], s.dtype)
    del dec
    d1 = layer.dims(1)
    for lay in layers:
        lay.workspace(max(mka.mka_workspace_bytes(d1, mka.MKA_OP_INDEX, nb0),
                          mka.mka_workspace_bytes(d1, mka.MKA_OP_DECODE_STEP, t_cap)))

    def reset():
        for lay in layers:
            lay.st["ema_state"].copy_(init["ema_state"])
            lay.st["block_acc"].copy_(init["block_acc"])
            lay.st["block_means"][:, :nb0].copy_(means0)
            lay.index_blocks(0, nb0)

    outs = [lay.outputs(1) for lay in layers]
    stream = torch.cuda.current_stream()

    def run(fn=None, n_copies=copies):
        """Two timed passes over the steps: one bracketed by two events alone
        (the throughput: recording an event between steps costs the GPU about
        2 us per step), then one with an event after every step (the per-step
        distribution).  Step k runs on copy k % n_copies at that copy's next
        position."""
        fns = [fn] if fn is not None else [lay.decode_step for lay in layers[:n_copies]]

        def steps_from_reset(evs=None):
            reset()
            for k in range(warmup):
                fns[k % n_copies](tokens[k], T0 + k // n_copies, out=outs[k % n_copies])
            reset()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record(stream)
            for k in range(steps):
                fns[k % n_copies](tokens[k], T0 + k // n_copies, out=outs[k % n_copies])
                if evs is not None:
                    evs[k].record(stream)
            e1.record(stream)
            host = (time.perf_counter() - t0) / steps * 1e6  # enqueue cost per step
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) / steps * 1e6
            return e0, e1, host, wall

        e0, e1, host_us, wall_us = steps_from_reset()
        mean_us = e0.elapsed_time(e1) * 1e3 / steps
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        f0, _, _, _ = steps_from_reset(ev)
        per_step = np.array([(f0 if k == 0 else ev[k - 1]).elapsed_time(ev[k]) * 1e3
                             for k in range(steps)])
        return mean_us, per_step, host_us, wall_us

    # Routing variants first (the same cache and state, the layer's shape
    # swapped); the main measurement runs last, from a reset state.
    var_us = {}
    for mode, tiers in variants:
        layer.shape = s.replace(route_mode=mode, tiers=tiers)
        var_us[f"{mode}/{tiers}"] = run(n_copies=1)[0]
        log(f"decode variant {mode}/{tiers}: {var_us[f'{mode}/{tiers}']:.1f} us/token")
    layer.shape = s
    full_us = None
    if full:
        f_us, _, f_host, _ = run(layer.full_decode_step, n_copies=1)
        full_us = {"us": f_us, "host_us": f_host}
        log(f"decode full MKA: {full_us['us']:.1f} us/token")
    mean_us, step_us, host_us, wall_us = run()
    warm = None
    if copies > 1:  # one layer re-read every step (its cache partly stays in the LLC)
        w_us, w_steps, w_host, _ = run(n_copies=1)
        warm = {"us": w_us, "median_us": float(np.median(w_steps)), "host_us": w_host}

    if page_size:  # the single-call attention entry takes contiguous caches
        return dict(us=mean_us, median_us=float(np.median(step_us)), host_us=host_us, cached=T0,
                    steps=steps)
    # Decode attention alone at the first step's length, for its roofline:
    # the copies' caches in turn (cold), and one cache re-read (warm).
    L = T0 + 1
    nbytes = mka.mka_workspace_bytes(d1, mka.MKA_OP_ATTN_DECODE, L)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(outs[0]["o"])
    reps = 48

    def attn_time(n_copies):
        def one(k):
            lay = layers[k % n_copies]
            mka.mka_attn_decode(d1, outs[k % n_copies]["q"], lay.st["k_cache"], lay.st["v_cache"],
                                t_cap, L, o, ws, nbytes, stream)
        for k in range(6):
            one(k)
        a_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        a_ev[0].record(stream)
        for k in range(reps):
            one(k)
        a_ev[1].record(stream)
        torch.cuda.synchronize()
        return a_ev[0].elapsed_time(a_ev[1]) * 1e3 / reps

    attn_us = attn_time(copies)
    attn_warm_us = attn_time(1) if copies > 1 else attn_us
    B = s.batch
    kv_bytes = 2.0 * L * s.n_kv_heads * s.head_dim * 2 * B  # K and V rows of every sequence, bf16
    el = 2
    # weights and hyperplanes once per step; cache rows, retrieved block rows and
    # block codes per sequence
    step_bytes = (kv_bytes + (s.q_width * s.d_model + 2 * s.kv_width * s.d_model
                              + s.router_hidden * s.q_width + 3 * s.router_hidden) * el
                  + s.hash_bits * s.d_model * 4 + B * (s.top_r * s.d_model * 4 + nb0 * 8))
    return dict(us=mean_us, median_us=float(np.median(step_us)), mean_us=float(step_us.mean()),
                wall_us=wall_us, host_us=host_us, attn_us=attn_us, attn_warm_us=attn_warm_us,
                kv_bytes=kv_bytes, step_bytes=step_bytes, cached=T0, steps=steps,
                variants_us=var_us, full=full_us, warm=warm, copies=copies)


def onbox_peaks():
    """Measured ceilings beside the published peaks: the library's dense bf16
    MFMA loop (two workgroups per CU, ~20 ms) and a streaming read of 4 GiB
    (beyond the last-level cache), each the median of 5 timed runs."""
    import torch

    from route_kv_memory_amd import mka

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    wg, iters = 2 * cus, 40000
    sink = torch.empty(max(wg, mka.PROBE_STREAM_WORKGROUPS), dtype=torch.float32, device="cuda")
    flops = wg * 4 * iters * 4 * 32768.0

    def timed(fn, reps=5):
        fn()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(out))

    t_mfma = timed(lambda: mka.mka_probe_mfma_bf16(wg, iters, sink, stream))
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    t_read = timed(lambda: mka.mka_probe_stream_read(buf, nbytes, sink, stream))
    del buf
    return {"mfma_bf16_tflops": flops / t_mfma / 1e12, "hbm_read_gbs": nbytes / t_read / 1e9,
            "note": "library probes: dense 32x32x16 bf16 MFMA loop (clocks drop under "
                    "sustained matrix load) and a 4 GiB streaming read"}


def host_info():
    """The host's CPU model, the threads the oracle's BLAS uses and the BLAS
    library numpy is built against."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    blas, threads = None, cores
    try:
        cfg = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{cfg.get('name')} {cfg.get('version')}"
    except Exception:  # noqa: BLE001 - build info is optional metadata
        pass
    try:
        from threadpoolctl import threadpool_info

        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            threads = pools[0]["num_threads"]
            blas = f"{pools[0].get('internal_api')} {pools[0].get('version')}"
    except Exception:  # noqa: BLE001
        pass
    return dict(cpu_model=model, cores=threads, host_cpus=cores, blas=blas)


def cpu_prefill(s, rows=None, n_tokens=None, batch=None):
    """The oracle, as it stands, on a prefill workload: every stage over every
    token (of the first ``n_tokens`` of ``batch`` sequences), attention on
    ``rows`` (every row when None).  Returns (seconds, description)."""
    from oracle import mka_oracle as O
    from route_kv_memory_amd.inputs import prefill_inputs

    batch = batch or s.batch
    n_tokens = n_tokens or s.seq
    inp = prefill_inputs(s.replace(batch=batch), seq=n_tokens)
    w = [inp[k] for k in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]
    kw = dict(n_heads=s.n_heads, n_kv_heads=s.n_kv_heads,
              ema_decay=float(np.float32(s.ema_decay)), block=s.block, top_r=s.top_r)
    t0 = time.perf_counter()
    O.prefill(inp["x"], *w, rows=rows, **kw)
    dt = time.perf_counter() - t0
    what = f"{batch}x{n_tokens} tokens of {s.name}, every stage over every token, attention "
    if rows is None:
        what += "on every row"
    else:
        n = len(rows)
        pairs = float(np.sum(np.asarray(rows) + 1))
        what += (f"on {n} sampled query rows ({100.0 * n / n_tokens:.2f}% of the rows, "
                 f"{100.0 * pairs / (n_tokens * (n_tokens + 1) / 2):.2f}% of the causal pairs)")
    return dt, what


def cpu_decode(s, attend_steps):
    """The oracle on the decode workload: every one of its steps on the carried
    state, attention at ``attend_steps`` only.  Returns (seconds, description)."""
    from oracle import mka_oracle as O
    from route_kv_memory_amd.inputs import decode_inputs

    dec = decode_inputs(s)
    w = [dec[k] for k in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]
    kw = dict(n_heads=s.n_heads, n_kv_heads=s.n_kv_heads,
              ema_decay=float(np.float32(s.ema_decay)), block=s.block, top_r=s.top_r)
    T0, n = s.decode_cached, s.decode_steps
    t0 = time.perf_counter()
    st = O.decode_init(dec["k_cache"], dec["v_cache"], dec["ema_state"], dec["block_acc"],
                       dec["block_means"], dec["proj"], t_cap=T0 + n)
    for k in range(n):
        O.decode_step(st, dec["tokens"][k], *w, attend=k in attend_steps, **kw)
    dt = time.perf_counter() - t0
    return dt, (f"{n} decode steps of {s.name} (state carried through every step, attention "
                f"at the {len(attend_steps)} steps {sorted(attend_steps)})")


def cpu_baselines(s_head, extra):
    """The oracle timed on bounded samples of every measured workload.  The
    headline entry is the one of the line's workload; the others are listed
    under ``workloads``."""
    from route_kv_memory_amd.inputs import sampled_rows, workload

    info = host_info()
    out = {}

    def prefill_entry(s):
        rows = sampled_rows(s) if s.n_sampled else None
        dt, what = cpu_prefill(s, rows=rows)
        log(f"cpu baseline {s.name}: {dt:.1f} s")
        return dict(value=s.batch * s.seq / dt, unit="tokens/s", seconds=dt,
                    kind="oracle (sampled)" if rows is not None else "oracle", sample=what)

    head = prefill_entry(s_head)
    for name in extra:
        s = workload(name)
        if s.is_decode:
            steps = {0, 1, 126, 127, 128, 129, 254, 255}
            dt, what = cpu_decode(s, steps)
            log(f"cpu baseline {s.name}: {dt:.1f} s")
            out[name] = dict(value=dt / s.decode_steps * 1e3, unit="ms/token",
                             seconds=dt, kind="oracle (attention on a step subset)", sample=what)
        else:
            out[name] = prefill_entry(s)
    line = dict(value=head["value"], unit="tokens/s", cores=info["cores"], kind="oracle",
                sample=f"{head['kind']}: {head['sample']}; fp64 NumPy, {head['seconds']:.1f} s",
                cpu_model=info["cpu_model"], host_cpus=info["host_cpus"], blas=info["blas"],
                workloads=out)
    return line


def prefill_entry(s, pf, onbox):
    """Figures of one timed prefill workload: tokens/s, the attention +
    projection fraction of bf16 MFMA peak and the attention kernel's roofline."""
    flops = prefill_flops(s)
    tokens = s.batch * s.seq
    stage_ms = pf["stage_ms"]
    achieved = flops["attn"] / (stage_ms["attn"] * 1e-3)
    return {
        "workload": s.name, "batch": s.batch, "seq_len": s.seq,
        "tokens_per_s": tokens / (pf["wall_ms"] * 1e-3), "ms_per_step": pf["wall_ms"],
        "gpu_ms_per_step": pf["gpu_ms"],
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "sequential_ms_per_step": pf["sequential_ms"],
        "flops": {k: v for k, v in flops.items()},
        "prefill_tflops": sum(flops.values()) / (pf["gpu_ms"] * 1e-3) / 1e12,
        "attn_proj_frac": sum(flops.values()) / (pf["gpu_ms"] * 1e-3) / PEAK_BF16_FLOPS,
        "roofline": {"kernel": ROOFLINE_KERNEL, "bound": "mfma", "achieved": achieved / 1e12,
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_FLOPS,
                     "traffic": traffic_for(ROOFLINE_KERNEL, s.name),
                     "onbox_peak": onbox["mfma_bf16_tflops"],
                     "frac_onbox": achieved / 1e12 / onbox["mfma_bf16_tflops"]},
    }


def decode_entry(ds, dc, onbox):
    """Figures of the timed decode workload: µs per token (cold: the copies in
    turn; warm: one layer re-read), the step's HBM fraction and the decode
    attention kernel's roofline."""
    attn_bw = dc["kv_bytes"] / (dc["attn_us"] * 1e-6)
    step_bw = dc["step_bytes"] / (dc["us"] * 1e-6)
    return {
        "workload": ds.name, "cached_tokens": dc["cached"], "steps": dc["steps"],
        "copies": dc["copies"],
        "copies_note": "the steps take the copies' layers (cache, weights, state) in turn, "
                       "so each step reads them from HBM (about 0.9 GB between two reads of "
                       "one copy, against a 256 MB last-level cache)",
        "us_per_token": dc["us"],
        "us_per_token_note": "GPU time of the steps between two events, over the steps; the "
                             "per-step figures come from a second pass with an event after "
                             "every step (each costs about 2 us)",
        "us_per_token_median": dc["median_us"], "us_per_token_mean": dc["mean_us"],
        "us_per_token_wall": dc["wall_us"], "us_per_token_host_enqueue": dc["host_us"],
        "step_bytes": dc["step_bytes"],
        "step_hbm_frac": step_bw / PEAK_HBM_BYTES,
        "warm": None if dc["warm"] is None else {
            "us_per_token": dc["warm"]["us"],
            "us_per_token_median": dc["warm"]["median_us"],
            "step_hbm_frac": dc["step_bytes"] / (dc["warm"]["us"] * 1e-6) / PEAK_HBM_BYTES,
            "attn_us_per_launch": dc["attn_warm_us"],
            "attn_hbm_frac": dc["kv_bytes"] / (dc["attn_warm_us"] * 1e-6) / PEAK_HBM_BYTES,
            "note": "one layer's cache and weights re-read every step (part of them stays "
                    "in the last-level cache)"},
        "roofline": {"kernel": "attn_decode", "bound": "hbm", "achieved": attn_bw / 1e9,
                     "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                     "frac": attn_bw / PEAK_HBM_BYTES,
                     "traffic": traffic_for("attn_decode_split_kernel", ds.name),
                     "us_per_launch": dc["attn_us"],
                     "onbox_peak": onbox["hbm_read_gbs"],
                     "frac_onbox": attn_bw / 1e9 / onbox["hbm_read_gbs"]},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_prefill_64k",
                    help="the headline prefill workload (the line's value and roofline)")
    ap.add_argument("--extra-workloads", default="qwen7b_prefill_4k,qwen7b_prefill_32k",
                    help="more prefill workloads reported under 'prefill' (comma list; '' none)")
    ap.add_argument("--aux-workload", default="qwen7b_prefill_4k",
                    help="the prefill workload of the training step, paged cache, full MKA and "
                         "routing variants")
    ap.add_argument("--decode-workload", default="qwen7b_decode_128k")
    ap.add_argument("--decode-copies", type=int, default=3,
                    help="layers (cache, weights, state) taken in turn by the decode steps")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="time the decode workload alone (for its counter passes); the line "
                         "then carries no prefill figures")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain copy of MIB MiB (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic file of --workload under profiles/ from two rocprofv3 "
                         "--pmc counter_collection.csv files (FETCH_SIZE, WRITE_SIZE); no GPU use")
    ap.add_argument("--traffic-workload", default=None,
                    help="with --traffic-summary: the workload the counters belong to (default "
                         "--workload)")
    ap.add_argument("--summary-command", action="append", default=[],
                    help="with --traffic-summary: the profiling commands, recorded verbatim")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed back-to-back prefill steps for this long before the warmup "
                         "(GPU clocks ramp up under load)")
    ap.add_argument("--full-mka", action="store_true",
                    help="also time full MKA (three attention paths mixed by lambda) on the "
                         "auxiliary workloads")
    ap.add_argument("--quick", action="store_true",
                    help="only the prefill and decode lines (skip the training step, paged "
                         "cache, batched decode, full MKA and routing variants that the default "
                         "run adds)")
    ap.add_argument("--train", action="store_true",
                    help="time a training step (forward with saved log-sum-exp, then the "
                         "backward) of the auxiliary workload (on by default)")
    ap.add_argument("--paged", type=int, default=0, metavar="ROWS",
                    help="time prefill and decode with a paged fused cache of pages of ROWS rows "
                         "(default 256 unless --quick)")
    ap.add_argument("--decode-batch", action="store_true",
                    help="time batched decode, 4 sequences of 32K cached tokens (on by default)")
    ap.add_argument("--variants", action="store_true",
                    help="also time the routing and tier variants (fixed, hard top-1/top-2; "
                         "L1+L2, L1+L3, L1 alone) on the auxiliary workloads")
    args = ap.parse_args()
    if not args.quick:  # every measured row of the build in the default line
        args.train = args.decode_batch = args.full_mka = args.variants = True
        args.paged = args.paged or 256
    if args.traffic_summary:
        res = traffic_summary(*args.traffic_summary, args.copy_calibration or 1024,
                              args.summary_command)
        res["workload"] = args.traffic_workload or args.workload
        with open(traffic_file(res["workload"]), "w") as fh:
            json.dump(res, fh, indent=1)
            fh.write("\n")
        print(json.dumps(res["kernels"], indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the FastMKA layer path here has no multi-GPU "
              "sharding (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from route_kv_memory_amd import inputs as I
    from route_kv_memory_amd import mka

    mka.lib()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    if args.decode_only:
        ds = I.workload(args.decode_workload)
        dc = bench_decode(ds, ds.decode_steps, 8, copies=max(1, args.decode_copies))
        print(json.dumps({"metric": METRIC, "n_gpus": 1, "data": "synthetic",
                          "decode": decode_entry(ds, dc, onbox_peaks())}), flush=True)
        return
    s = I.workload(args.workload)
    extra = [w for w in args.extra_workloads.split(",") if w]
    variants = VARIANTS if args.variants else ()
    aux = args.aux_workload
    # the headline workload (and, when it is also the auxiliary one, its variants)
    pf = bench_prefill(s, args.steps, args.warmup, variants if s.name == aux else (),
                       args.settle_ms, args.full_mka and s.name == aux)
    log(f"prefill {s.name}: {pf['wall_ms']:.3f} ms per step, attention {pf['stage_ms']['attn']:.3f} ms")
    onbox = onbox_peaks()
    log(f"on-box peaks: {onbox['mfma_bf16_tflops']:.0f} TFLOP/s bf16 MFMA, "
        f"{onbox['hbm_read_gbs']:.0f} GB/s streaming read")
    head = prefill_entry(s, pf, onbox)
    tokens = s.batch * s.seq
    ms = pf["wall_ms"]
    line = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) hiddens, N(0,1/d_in) weights)",
        "config": {"workload": s.name, "batch": s.batch, "seq_len": s.seq, "d_model": s.d_model,
                   "n_heads": s.n_heads, "n_kv_heads": s.n_kv_heads, "head_dim": s.head_dim,
                   "block": s.block, "top_r": s.top_r, "hash_bits": s.hash_bits},
        "gpu_ms_per_step": pf["gpu_ms"],
        "settle": {"ms": args.settle_ms, "steps": pf["settle_steps"],
                   "note": "untimed back-to-back steps before the warmup, so that the timed "
                           "steps run at the clocks of a loaded GPU"},
        "stages_ms": head["stages_ms"],
        "stages_note": "stage calls one by one on one stream (the timed composite overlaps the "
                       "ema/index/retrieve chain with route)",
        "sequential_ms_per_step": pf["sequential_ms"],
        "prefill_tflops": head["prefill_tflops"],
        "attn_proj_frac": head["attn_proj_frac"],
        "roofline": head["roofline"],
        "onbox_peaks": onbox,
        "prefill": {},
    }
    pf_aux = pf if s.name == aux else None
    for name in extra:
        sw = I.workload(name)
        pfw = bench_prefill(sw, args.steps, args.warmup, variants if name == aux else (),
                            args.settle_ms, args.full_mka and name == aux)
        log(f"prefill {name}: {pfw['wall_ms']:.3f} ms per step, attention "
            f"{pfw['stage_ms']['attn']:.3f} ms")
        line["prefill"][name] = prefill_entry(sw, pfw, onbox)
        if name == aux:
            pf_aux = pfw
    s_aux = I.workload(aux)
    aux_tokens = s_aux.batch * s_aux.seq
    dc = None
    if not args.no_decode:
        ds = I.workload(args.decode_workload)
        dc = bench_decode(ds, ds.decode_steps, 8, variants, args.full_mka,
                          copies=max(1, args.decode_copies))
        line["decode"] = decode_entry(ds, dc, onbox)
    if variants and pf_aux is not None:
        line["variants"] = {
            k: {"workload": aux, "prefill_tokens_per_s": aux_tokens / (v * 1e-3), "prefill_ms": v,
                "decode_us_per_token": dc["variants_us"].get(k) if dc else None}
            for k, v in pf_aux["variants_ms"].items()}
    if args.train:
        tr = bench_train(s_aux, args.steps, args.warmup, args.settle_ms)
        log(f"training step: {tr['ms']:.3f} ms (forward {tr['fwd_ms']:.3f}, backward "
            f"{tr['bwd_ms']:.3f})")
        # the four products of the attention gradient (dV, dP, dQ, dK), 2*dh flops
        # per causal pair each; recomputing the scores is not counted
        bwd_flops = 2.0 * prefill_flops(s_aux)["attn"]
        bwd_ach = bwd_flops / (tr["attn_bwd_ms"] * 1e-3)
        line["train"] = {"workload": aux, "tokens_per_s": aux_tokens / (tr["ms"] * 1e-3),
                         "ms_per_step": tr["ms"],
                         "forward_ms": tr["fwd_ms"], "backward_ms": tr["bwd_ms"],
                         "attn_backward_ms": tr["attn_bwd_ms"],
                         "roofline": {"kernel": "attn_bwd_dkv_kernel + attn_bwd_dq_kernel",
                                      "bound": "mfma", "achieved": bwd_ach / 1e12,
                                      "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                                      "frac": bwd_ach / PEAK_BF16_FLOPS,
                                      "onbox_peak": onbox["mfma_bf16_tflops"],
                                      "frac_onbox": bwd_ach / 1e12 / onbox["mfma_bf16_tflops"]},
                         "note": "mka_prefill (saving log-sum-exp) + mka_backward: gradients of "
                                 "x and every weight, fp32"}
    if args.paged:
        pms = bench_prefill_paged(s_aux, args.steps, args.warmup, args.paged, args.settle_ms)
        log(f"paged prefill (pages of {args.paged}): {pms:.4f} ms")
        line["paged"] = {"workload": aux, "page_size": args.paged, "prefill_ms": pms,
                         "prefill_tokens_per_s": aux_tokens / (pms * 1e-3)}
        if not args.no_decode:
            ds = I.workload(args.decode_workload)
            pdc = bench_decode(ds, ds.decode_steps, 8, page_size=args.paged)
            log(f"paged decode: {pdc['us']:.1f} us/token")
            line["paged"].update(decode_us_per_token=pdc["us"],
                                 decode_host_us_per_token=pdc["host_us"],
                                 decode_note="one layer re-read every step (compare decode.warm)")
    if args.decode_batch:
        bs = I.workload("qwen7b_decode_32k_b4")
        bdc = bench_decode(bs, bs.decode_steps, 8)
        log(f"batched decode B={bs.batch}: {bdc['us']:.1f} us/step")
        line["decode_batch"] = {
            "workload": bs.name, "batch": bs.batch, "cached_tokens": bdc["cached"],
            "us_per_step": bdc["us"], "us_per_step_median": bdc["median_us"],
            "tokens_per_s": bs.batch / (bdc["us"] * 1e-6),
            "step_hbm_frac": bdc["step_bytes"] / (bdc["us"] * 1e-6) / PEAK_HBM_BYTES,
            "attn_us_per_launch": bdc["attn_us"],
            "attn_hbm_frac": bdc["kv_bytes"] / (bdc["attn_us"] * 1e-6) / PEAK_HBM_BYTES,
            "note": "one layer re-read every step (its 4 x 32K cache is 269 MB)"}
    if args.full_mka and pf_aux is not None and pf_aux["full_ms"] is not None:
        line["full_mka"] = {
            "workload": aux,
            "prefill_ms": pf_aux["full_ms"],
            "prefill_tokens_per_s": aux_tokens / (pf_aux["full_ms"] * 1e-3),
            "decode_us_per_token": dc["full"]["us"] if dc else None,
            "decode_host_us_per_token": dc["full"]["host_us"] if dc else None,
            "note": "three attention paths (one K/V cache per tier) mixed by lambda; same "
                    "inputs as the FastMKA figures of this line; decode on one layer re-read"}
    if not args.no_cpu_baseline:
        log("cpu baseline: the oracle on bounded samples")
        others = [w for w in ["tiny_f32"] + extra + [args.decode_workload] if w != s.name]
        line["cpu_baseline"] = cpu_baselines(s, others)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

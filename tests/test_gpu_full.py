"""GPU parity at the workloads' full sizes, against the oracle.

Prefill: the Qwen2.5-7B-shaped layer at 4096 tokens x 2 sequences and at
32768 tokens (with drift), and the Llama-3.1-8B-shaped layer at 65536
tokens.  The oracle computes every step for every row (later rows need the
earlier ones) and attention on sampled rows; router weights, L2, block
means, codes and retrieved blocks are compared on every row, Q/K/V/O on the
sampled rows.  Decode: the 131072-token fused-cache workload, 256 steps,
compared at sampled steps and on the final state.  Backward: the 4096-token
workload's training step, every gradient against the oracle's chain rule.
The launch configuration is the one bench.py times.
"""

import gc

import numpy as np
import pytest
import torch

from oracle import mka_oracle as O
from route_kv_memory_amd import inputs as I
from route_kv_memory_amd import mka
from route_kv_memory_amd.layer import Layer, to_device

from .gpu_common import to_np
from .parity import (check_close, check_codes, check_idx, check_idx_conditional, log,
                     oracle_kwargs)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

WEIGHTS = ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")


def _rows(s):
    if s.n_sampled:
        return I.sampled_rows(s)
    return I.sampled_rows(s.replace(n_sampled=512))


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["qwen7b_prefill_4k", "qwen7b_prefill_32k", "llama8b_prefill_64k"])
def test_full_prefill(name):
    s = I.workload(name)
    log(f"[{name}] generating inputs")
    inp = I.prefill_inputs(s)
    rows = _rows(s)
    N, B = s.seq, s.batch
    layer = Layer(s, inp, t_cap=N, nb_cap=N // s.block)
    log(f"[{name}] gpu: mka_prefill B={B} N={N}")
    out = layer.prefill(to_device(inp["x"], s.dtype))
    torch.cuda.synchronize()
    g = {
        "lam": to_np(out["lambda"]),
        "key": to_np(out["key"]).view(np.uint64),
        "idx": to_np(out["idx"]),
        "l2": to_np(out["l2"]),
        "q": to_np(out["q"][:, rows]).reshape(B, len(rows), -1),
        "o": to_np(out["o"][:, rows]),
        "k": to_np(layer.st["k_cache"][:, :, rows]),
        "v": to_np(layer.st["v_cache"][:, :, rows]),
        "means": to_np(layer.st["block_means"]),
        "bhash": to_np(layer.st["block_hash"]).view(np.uint64),
    }
    del out, layer
    torch.cuda.empty_cache()
    log(f"[{name}] oracle (every step on every row, attention on {len(rows)} rows)")
    ref = O.prefill(inp["x"], *[inp[k] for k in WEIGHTS], rows=rows, **oracle_kwargs(s))
    check_close("lambda", g["lam"], ref["lam"], s.dtype)
    check_close("l2 (sampled rows)", g["l2"][:, rows], ref["l2"][:, rows], "f32")
    check_close("block_means", g["means"], ref["block_means"], "f32")
    check_codes("block_hash", g["bhash"], ref["block_hash"], ref["block_abs"], s.hash_bits)
    check_codes("keys", g["key"], ref["keys"], ref["key_abs"], s.hash_bits)
    check_idx("idx", g["idx"], ref["keys"], ref["key_abs"], ref["block_hash"], ref["block_abs"],
              np.arange(N), s.block, s.top_r, s.hash_bits)
    check_idx_conditional("idx|gpu", g["idx"], g["key"], g["l2"], g["means"], g["bhash"],
                          inp["proj"], np.arange(N), s.block, s.top_r, s.hash_bits)
    check_close("q (sampled rows)", g["q"], ref["q"][:, rows], s.dtype)
    check_close("k (sampled rows)", g["k"], ref["k"][:, :, rows], s.dtype)
    check_close("v (sampled rows)", g["v"], ref["v"][:, :, rows], s.dtype)
    check_close("o (sampled rows)", g["o"], ref["o"], s.dtype)
    del ref, g, inp
    gc.collect()


@pytest.mark.timeout(1200)
def test_full_decode_128k():
    s = I.workload("qwen7b_decode_128k")
    log("[decode] generating state")
    dec = I.decode_inputs(s)
    T0, n = s.decode_cached, s.decode_steps
    t_cap = T0 + n
    nb0 = T0 // s.block
    sample = {0, 1, 126, 127, 128, 129, 254, 255}
    layer = Layer(s, dec, t_cap=t_cap, nb_cap=t_cap // s.block + 1)
    st = layer.st
    st["k_cache"][:, :, :T0] = to_device(dec["k_cache"], s.dtype)
    st["v_cache"][:, :, :T0] = to_device(dec["v_cache"], s.dtype)
    st["ema_state"].copy_(to_device(dec["ema_state"]))
    st["block_acc"].copy_(to_device(dec["block_acc"]))
    st["block_means"][:, :nb0].copy_(to_device(dec["block_means"]))
    d1 = layer.dims(1)
    ws = layer.workspace(max(mka.mka_workspace_bytes(d1, mka.MKA_OP_INDEX, nb0),
                             mka.mka_workspace_bytes(d1, mka.MKA_OP_DECODE_STEP, t_cap)))
    layer.index_blocks(0, nb0)
    tokens = to_device(dec["tokens"], s.dtype)
    log(f"[decode] gpu: {n} mka_decode_step calls from position {T0}")
    got = {}
    for k in range(n):
        out = layer.decode_step(tokens[k], T0 + k)
        if k in sample:
            torch.cuda.synchronize()
            got[k] = {kk: to_np(v) for kk, v in out.items()}
            got[k]["key"] = got[k]["key"].view(np.uint64)
    torch.cuda.synchronize()
    fin = {"k": to_np(st["k_cache"][:, :, T0:]), "v": to_np(st["v_cache"][:, :, T0:]),
           "means": to_np(st["block_means"][:, :nb0 + 2]),
           "bhash": to_np(st["block_hash"][:, :nb0 + 2]).view(np.uint64)}
    del layer, st, tokens
    torch.cuda.empty_cache()

    log("[decode] oracle: 256 steps of state, attention at the sampled steps")
    w = [dec[k] for k in WEIGHTS]
    kw = oracle_kwargs(s)
    ost = O.decode_init(dec["k_cache"], dec["v_cache"], dec["ema_state"], dec["block_acc"],
                        dec["block_means"], dec["proj"], t_cap=t_cap)
    for k in range(n):
        r = O.decode_step(ost, dec["tokens"][k], *w, attend=k in sample, **kw)
        if k in sample:
            gk = got[k]
            log(f"  step {k} (position {T0 + k})")
            check_close("o", gk["o"][:, 0], r["o"], s.dtype)
            check_close("lambda", gk["lambda"][:, 0], r["lam"], s.dtype)
            check_close("l2", gk["l2"][:, 0], r["l2"], "f32")
            check_codes("key", gk["key"][:, 0], r["key"], r["key_abs"], s.hash_bits)
            check_idx("idx", gk["idx"], r["key"][:, None], r["key_abs"][:, None], ost.hash,
                      ost.hash_abs, np.array([T0 + k]), s.block, s.top_r, s.hash_bits)
    check_close("k rows appended", fin["k"], ost.k[:, :, T0:], s.dtype)
    check_close("v rows appended", fin["v"], ost.v[:, :, T0:], s.dtype)
    check_close("block means (incl. the two completed)", fin["means"], ost.means, "f32")
    check_codes("block codes (incl. the two completed)", fin["bhash"], ost.hash, ost.hash_abs,
                s.hash_bits)


@pytest.mark.timeout(1200)
def test_full_backward_4k():
    """mka_prefill + mka_backward, and mka_attn_backward alone, at the 2 x 4096-token
    Qwen2.5-7B-shaped workload in the launch configuration of the timed training step.

    The loss is sum(O * dO) with dO = 0 on the first sequence, so every gradient is
    the second sequence's alone: the oracle runs the fp64 chain rule on that sequence
    (every row, every head), and the first sequence's dx must be exactly zero."""
    from .test_gpu_backward import check_grad

    s = I.workload("qwen7b_prefill_4k")
    B, N, H, G, dh = s.batch, s.seq, s.n_heads, s.n_kv_heads, s.head_dim
    log("[backward 4k] generating inputs")
    inp = I.prefill_inputs(s)
    d_o = np.zeros((B, N, H, dh), np.float32)
    d_o[1] = I.round_bf16(np.random.default_rng(101).standard_normal((N, H, dh)))
    layer = Layer(s, inp, t_cap=N, nb_cap=N // s.block)
    x = to_device(inp["x"], s.dtype)
    d_o_dev = to_device(d_o, s.dtype)
    log(f"[backward 4k] gpu: mka_prefill + mka_backward B={B} N={N}")
    out = layer.prefill(x)
    g = layer.backward(x, out, d_o_dev)
    d = layer.dims(N)
    dq = torch.empty(B, N, H, dh, device="cuda")
    dkv = torch.empty(B, N, 2, G, dh, device="cuda")
    ws = torch.empty(max(256, mka.mka_workspace_bytes(d, mka.MKA_OP_ATTN_BACKWARD)),
                     dtype=torch.uint8, device="cuda")
    log("[backward 4k] gpu: mka_attn_backward")
    mka.mka_attn_backward(d, out["q"], layer.st["k_cache"], layer.st["v_cache"], layer.t_cap,
                          out["o"], out["lse"], d_o_dev, dq, dkv, ws, ws.numel())
    torch.cuda.synchronize()
    got = {k: to_np(v) for k, v in g.items()}
    a_dkv = to_np(dkv)
    lse = to_np(out["lse"])
    idx = to_np(out["idx"])
    del out, layer, x, d_o_dev, dq, dkv, ws, g
    torch.cuda.empty_cache()

    assert np.all(got["dx"][0] == 0.0), "dO = 0 on a sequence must give it dx = 0"
    assert np.all(a_dkv[0] == 0.0), "dO = 0 on a sequence must give it dK = dV = 0"
    log("[backward 4k] oracle: forward and chain rule on the second sequence")
    ref = O.backward(inp["x"][1:2], *[inp[k] for k in WEIGHTS], d_o[1:2], **oracle_kwargs(s))
    n_diff = int(np.sum(np.any(idx[1] != ref["fwd"]["idx"][0], axis=-1)))
    log(f"  rows whose retrieved blocks differ from the oracle's (code near-ties): {n_diff}")
    # the saved log-sum-exp on sampled rows, from the oracle's own q and K
    qh = ref["fwd"]["q"][0].reshape(N, H, dh)
    rows = I.sampled_rows(s.replace(n_sampled=64))
    want = np.empty((len(rows), H))
    for i, t in enumerate(rows):
        for h in range(H):
            sc = ref["fwd"]["k"][0, h // (H // G), :t + 1] @ qh[t, h] / np.sqrt(dh)
            want[i, h] = sc.max() + np.log(np.exp(sc - sc.max()).sum())
    check_close("lse (sampled rows)", lse[1, rows], want, s.dtype)
    check_grad("dx", got["dx"][1], ref["dx"][0], s.dtype)
    for k in ("dw_q", "dw_k", "dw_v", "dw_r1", "dw_r2"):
        check_grad(k, got[k], ref[k], s.dtype)
    check_grad("attn dk", a_dkv[1, :, 0].transpose(1, 0, 2), ref["dk"][0], s.dtype)
    check_grad("attn dv", a_dkv[1, :, 1].transpose(1, 0, 2), ref["dv"][0], s.dtype)
    del ref, got, inp
    gc.collect()


def _bitwise_equal(name, a, b):
    a, b = to_np(a), to_np(b)
    assert a.shape == b.shape, (name, a.shape, b.shape)
    same = np.array_equal(a.view(np.uint8), b.view(np.uint8))
    log(f"  {name}: {'bit-identical' if same else 'DIFFERS'}")
    assert same, f"{name}: paged and contiguous layers differ"


@pytest.mark.timeout(1200)
def test_full_paged_matches_contiguous():
    """The paged fused cache at full size, in the launch configuration the bench
    times (256-row pages in a seeded random order, spare pages in the pool):
    2 x 4096 prefill and 16 decode steps at 131072 cached tokens give outputs and
    cache rows bit-identical to the contiguous layer (only addresses differ; both
    are checked against the oracle at these sizes by the tests above)."""
    s = I.workload("qwen7b_prefill_4k")
    log("[paged 4k] generating inputs")
    inp = I.prefill_inputs(s)
    x = to_device(inp["x"], s.dtype)
    res = {}
    for name, kw in (("contiguous", {}), ("paged", dict(page_size=256, spare_pages=8))):
        layer = Layer(s, inp, t_cap=s.seq, nb_cap=s.seq // s.block, **kw)
        log(f"[paged 4k] gpu: mka_prefill, {name}")
        out = layer.prefill(x)
        torch.cuda.synchronize()
        res[name] = (out, layer.logical_cache("k")[:, :, :s.seq].clone(),
                     layer.logical_cache("v")[:, :, :s.seq].clone())
        del layer
    for key in ("q", "lambda", "l2", "key", "idx", "o", "lse"):
        _bitwise_equal(f"prefill {key}", res["contiguous"][0][key], res["paged"][0][key])
    _bitwise_equal("prefill K cache", res["contiguous"][1], res["paged"][1])
    _bitwise_equal("prefill V cache", res["contiguous"][2], res["paged"][2])
    del res, x, inp
    torch.cuda.empty_cache()

    s = I.workload("qwen7b_decode_128k")
    log("[paged 128k] generating state")
    dec = I.decode_inputs(s)
    T0, n = s.decode_cached, 16
    t_cap = T0 + s.decode_steps
    nb0 = T0 // s.block
    tokens = to_device(dec["tokens"], s.dtype)
    res = {}
    for name, kw in (("contiguous", {}), ("paged", dict(page_size=256, spare_pages=8))):
        layer = Layer(s, dec, t_cap=t_cap, nb_cap=t_cap // s.block + 1, **kw)
        st = layer.st
        layer.load_cache("k", to_device(dec["k_cache"], s.dtype))
        layer.load_cache("v", to_device(dec["v_cache"], s.dtype))
        st["ema_state"].copy_(to_device(dec["ema_state"]))
        st["block_acc"].copy_(to_device(dec["block_acc"]))
        st["block_means"][:, :nb0].copy_(to_device(dec["block_means"]))
        d1 = layer.dims(1)
        layer.workspace(max(mka.mka_workspace_bytes(d1, mka.MKA_OP_INDEX, nb0),
                            mka.mka_workspace_bytes(d1, mka.MKA_OP_DECODE_STEP, t_cap)))
        layer.index_blocks(0, nb0)
        log(f"[paged 128k] gpu: {n} mka_decode_step calls from position {T0}, {name}")
        outs = []
        for k in range(n):
            out = layer.decode_step(tokens[k], T0 + k)
            outs.append({kk: v.clone() for kk, v in out.items()})
        torch.cuda.synchronize()
        res[name] = (outs, layer.logical_cache("k")[:, :, T0:T0 + n].clone(),
                     layer.logical_cache("v")[:, :, T0:T0 + n].clone())
        del layer, st
        torch.cuda.empty_cache()
    for k in range(n):
        for key in ("lambda", "l2", "key", "idx", "o"):
            _bitwise_equal(f"decode step {k} {key}", res["contiguous"][0][k][key],
                           res["paged"][0][k][key])
    _bitwise_equal("decode K rows appended", res["contiguous"][1], res["paged"][1])
    _bitwise_equal("decode V rows appended", res["contiguous"][2], res["paged"][2])

"""GPU parity of the whole FastMKA layer on small shapes, against the oracle.

Every check goes through the C ABI.  Shapes: the tiny fp32 layer (D=128,
2 query / 1 KV head of 64, block 64, 32-bit codes, R=2), the same layer in
bf16, and a small bf16 layer with 128-wide heads and a ragged length.
"""

import numpy as np
import pytest
import torch

from oracle import mka_oracle as O
from route_kv_memory_amd import inputs as I
from route_kv_memory_amd import mka
from route_kv_memory_amd.layer import Layer, to_device

from .gpu_common import gpu_prefill, outputs_np, state_np, to_np
from .parity import (check_close, check_codes, check_idx, check_idx_conditional, log,
                     oracle_kwargs)

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_f32": I.workload("tiny_f32"),
    "tiny_bf16": I.workload("tiny_f32").replace(name="tiny_bf16", dtype="bf16"),
    "small_bf16_dh128": I.workload("tiny_f32").replace(
        name="small_bf16_dh128", dtype="bf16", seq=333, d_model=256, n_heads=4, n_kv_heads=2,
        head_dim=128, router_hidden=64, block=32, hash_bits=64, top_r=4, ema_decay=0.95, seed=11),
    "small_f32_b2": I.workload("tiny_f32").replace(
        name="small_f32_b2", batch=2, seq=200, d_model=64, n_heads=4, n_kv_heads=2,
        head_dim=64, router_hidden=16, block=16, hash_bits=64, top_r=5, seed=12),
}


def oracle_for(s, inp, rows=None):
    w = [inp[k] for k in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]
    return O.prefill(inp["x"], *w, rows=rows, **oracle_kwargs(s))


def compare_layer(s, proj, ref, out, st, rows=None):
    B, N = ref["lam"].shape[:2]
    rows = np.arange(N) if rows is None else rows
    check_close("q", out["q"].reshape(B, N, -1), ref["q"], s.dtype)
    check_close("lambda", out["lambda"], ref["lam"], s.dtype)
    check_close("l2", out["l2"], ref["l2"], "f32")
    nb = ref["block_means"].shape[1]
    if nb:
        check_close("block_means", st["means"][:, :nb], ref["block_means"], "f32")
        check_codes("block_hash", st["bhash"][:, :nb], ref["block_hash"], ref["block_abs"], s.hash_bits)
    check_codes("keys", out["key"], ref["keys"], ref["key_abs"], s.hash_bits)
    check_idx("idx", out["idx"], ref["keys"], ref["key_abs"], ref["block_hash"], ref["block_abs"],
              np.arange(N), s.block, s.top_r, s.hash_bits)
    if nb:
        check_idx_conditional("idx|gpu", out["idx"], out["key"], out["l2"], st["means"][:, :nb],
                              st["bhash"][:, :nb], proj, np.arange(N), s.block,
                              s.top_r, s.hash_bits)
    check_close("k", st["k"][:, :, :N], ref["k"], s.dtype)
    check_close("v", st["v"][:, :, :N], ref["v"], s.dtype)
    check_close("o", out["o"][:, rows], ref["o"], s.dtype)



@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_prefill(name):
    s = SMALL[name]
    inp = I.prefill_inputs(s)
    ref = oracle_for(s, inp)
    layer, out = gpu_prefill(s, inp)
    compare_layer(s, inp["proj"], ref, outputs_np(out), state_np(layer))
    st = state_np(layer)
    check_close("ema_state", st["ema"], ref["l2"][:, -1], "f32")
    # projected block means: row b = m_b [W_k; W_v]^T, recomputed in float64 from
    # the GPU's own block means (a property of the kept rows, at any size)
    nb = ref["block_means"].shape[1]
    if nb:
        w_kv = np.concatenate([inp["w_k"], inp["w_v"]], axis=0).astype(np.float64)
        want = st["means"][:, :nb].astype(np.float64) @ w_kv.T
        check_close("block_kv", st["block_kv"][:, :nb], want, "f32")


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16_dh128"])
def test_chunked_prefill_equals_whole(name):
    # prefill(0..k) then prefill(k..N) at pos0 = k leaves the same state and outputs.
    s = SMALL[name]
    inp = I.prefill_inputs(s)
    N, k = s.seq, 100
    whole_layer, whole = gpu_prefill(s, inp)
    layer = Layer(s, inp, t_cap=N, nb_cap=max(1, N // s.block))
    gpu_prefill(s, inp, x=inp["x"][:, :k], layer=layer)
    _, second = gpu_prefill(s, inp, x=inp["x"][:, k:], layer=layer, pos0=k)
    w, c = outputs_np(whole), outputs_np(second)
    for key in ("lambda", "l2", "idx", "key", "o", "q"):
        tol = 1e-6 if s.dtype == "f32" else 1e-2
        np.testing.assert_allclose(np.asarray(c[key], np.float64),
                                   np.asarray(w[key][:, k:], np.float64), atol=tol, err_msg=key)
    ws, cs = state_np(whole_layer), state_np(layer)
    np.testing.assert_allclose(cs["means"], ws["means"], atol=1e-6)
    np.testing.assert_array_equal(cs["bhash"], ws["bhash"])
    np.testing.assert_allclose(cs["k"], ws["k"], atol=1e-5 if s.dtype == "f32" else 1e-2)


@pytest.mark.parametrize("name,n1", [("tiny_f32", 128), ("small_bf16_dh128", 190),
                                     ("tiny_bf16", 1)])
def test_decode_continues_prefill(name, n1):
    # prefill(n1) then one mka_decode_step per token == prefill of the whole
    # sequence, across block completions (bf16: the overlapped two-stream step).
    s = SMALL[name]
    inp = I.prefill_inputs(s)
    ref = oracle_for(s, inp)
    layer = Layer(s, inp, t_cap=s.seq, nb_cap=s.seq // s.block)
    gpu_prefill(s, inp, x=inp["x"][:, :n1], layer=layer)
    xs = to_device(inp["x"], s.dtype)
    log(f"  gpu: {s.seq - n1} mka_decode_step calls")
    outs = []
    for t in range(n1, s.seq):
        out = layer.decode_step(xs[:, t:t + 1].contiguous(), t)
        outs.append(outputs_np(out))
    torch.cuda.synchronize()
    o = np.concatenate([r["o"] for r in outs], axis=1)
    check_close("decode o", o, ref["o"][:, n1:], s.dtype)
    check_close("decode lambda", np.concatenate([r["lambda"] for r in outs], 1), ref["lam"][:, n1:],
                s.dtype)
    check_close("decode l2", np.concatenate([r["l2"] for r in outs], 1), ref["l2"][:, n1:], "f32")
    idx = np.concatenate([r["idx"] for r in outs], 1)
    check_idx("decode idx", idx, ref["keys"][:, n1:], ref["key_abs"][:, n1:], ref["block_hash"],
              ref["block_abs"], np.arange(n1, s.seq), s.block, s.top_r, s.hash_bits)
    st = state_np(layer)
    check_close("decode k", st["k"], ref["k"], s.dtype)
    check_close("decode v", st["v"], ref["v"], s.dtype)
    nb = ref["block_means"].shape[1]
    check_close("decode block means", st["means"][:, :nb], ref["block_means"], "f32")
    check_codes("decode block_hash", st["bhash"][:, :nb], ref["block_hash"], ref["block_abs"],
                s.hash_bits)


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_bf16", "small_bf16_dh128"])
def test_one_hot_router_is_causal_gqa(name):
    # lambda forced to (1, 0, 0) through mka_fuse_kv_proj: the layer reduces to
    # standard causal GQA attention of X W_q against X W_k, X W_v.
    s = SMALL[name]
    inp = I.prefill_inputs(s)
    B, N, D = s.batch, s.seq, s.d_model
    lam = np.zeros((B, N, 3), np.float32)
    lam[..., 0] = 1.0
    ref = O.prefill(inp["x"], *[inp[k] for k in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")],
                    lam_override=lam, **oracle_kwargs(s))
    layer, out = gpu_prefill(s, inp)  # fills l2, idx, block means
    d = mka.dims(s)
    ws = layer.workspace(mka.mka_workspace_bytes(d, mka.MKA_OP_FUSE_KV))
    mka.mka_fuse_kv_proj(d, to_device(inp["x"], s.dtype), out["l2"], layer.st["block_means"],
                         layer.nb_cap, out["idx"], torch.from_numpy(lam).cuda(), layer.w["w_k"],
                         layer.w["w_v"], layer.st["k_cache"], layer.st["v_cache"], 0, layer.t_cap,
                         ws, ws.numel())
    o = torch.empty_like(out["o"])
    mka.mka_attn_prefill(d, out["q"], layer.st["k_cache"], layer.st["v_cache"], layer.t_cap, 0, o)
    torch.cuda.synchronize()
    check_close("k one-hot", to_np(layer.st["k_cache"]), ref["k"], s.dtype)
    check_close("o one-hot", to_np(o), ref["o"], s.dtype)


def test_gpu_layer_is_causal_and_deterministic():
    s = SMALL["small_bf16_dh128"]
    inp = I.prefill_inputs(s)
    _, a = gpu_prefill(s, inp)
    _, a2 = gpu_prefill(s, inp)
    a, a2 = outputs_np(a), outputs_np(a2)
    for key in a:
        np.testing.assert_array_equal(a[key], a2[key], err_msg=f"run-to-run {key}")
    t0 = 150
    x2 = inp["x"].copy()
    x2[:, t0 + 1:] = I.round_bf16(np.random.default_rng(99).standard_normal(x2[:, t0 + 1:].shape))
    _, b = gpu_prefill(s, inp, x=x2)
    b = outputs_np(b)
    for key in a:
        np.testing.assert_array_equal(a[key][:, : t0 + 1], b[key][:, : t0 + 1], err_msg=key)
    assert not np.array_equal(a["o"][:, t0 + 1:], b["o"][:, t0 + 1:])


def test_isolated_attention_bf16_tight():
    # Attention alone on oracle-provided bf16 Q/K/V: only the kernel's own
    # rounding (P in bf16, fp32 accumulation) separates it from the oracle.
    s = SMALL["small_bf16_dh128"]
    r = np.random.default_rng(5)
    B, N, H, G, dh = 1, 517, s.n_heads, s.n_kv_heads, s.head_dim
    q = I.round_bf16(r.standard_normal((B, N, H, dh)))
    k = I.round_bf16(r.standard_normal((B, G, N, dh)))
    v = I.round_bf16(r.standard_normal((B, G, N, dh)))
    rows = np.arange(N)
    ref = O.attention(q, k, v, rows, G)
    d = mka.dims(s, seq=N, batch=B)
    o = torch.empty(B, N, H, dh, dtype=torch.bfloat16, device="cuda")
    mka.mka_attn_prefill(d, to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"), N, 0, o)
    torch.cuda.synchronize()
    check_close("attn isolated", to_np(o), ref, "bf16", max_abs=1e-2, mean_abs=1e-3)


def test_decode_attention_matches_prefill_row():
    # mka_attn_decode at cache length L equals the causal attention of the
    # query at position L-1 (split over 1024-key chunks, ragged last chunk).
    s = SMALL["small_bf16_dh128"]
    r = np.random.default_rng(6)
    B, H, G, dh = 1, s.n_heads, s.n_kv_heads, s.head_dim
    for L in (1, 63, 1024, 1025, 3000):
        q = I.round_bf16(r.standard_normal((B, 1, H, dh)))
        k = I.round_bf16(r.standard_normal((B, G, L, dh)))
        v = I.round_bf16(r.standard_normal((B, G, L, dh)))
        ref = O.attention(q, k, v, np.array([L - 1]), G)
        d = mka.dims(s, seq=1, batch=B)
        nbytes = mka.mka_workspace_bytes(d, mka.MKA_OP_ATTN_DECODE, L)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        o = torch.empty(B, 1, H, dh, dtype=torch.bfloat16, device="cuda")
        log(f"  gpu: mka_attn_decode L={L}")
        mka.mka_attn_decode(d, to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"), L,
                            L, o, ws, ws.numel())
        torch.cuda.synchronize()
        check_close(f"decode attn L={L}", to_np(o), ref, "bf16", max_abs=1e-2, mean_abs=1e-3)


def test_peak_probes_run():
    # The measurement probes complete and write their sinks (values carry no meaning).
    sink = torch.full((mka.PROBE_STREAM_WORKGROUPS,), float("nan"), device="cuda")
    mka.mka_probe_mfma_bf16(8, 16, sink)
    torch.cuda.synchronize()
    assert torch.isfinite(sink[:8]).all()
    buf = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    mka.mka_probe_stream_read(buf, buf.numel() * 4, sink)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()

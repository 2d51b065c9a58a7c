"""GPU parity of the layer backward (mka_backward) against the oracle.

After mka_prefill over a whole sequence (which also writes each query row's
log-sum-exp), mka_backward gives the float32 gradients of sum(O * dO) with
respect to x, W_q, W_k, W_v, W_r1 and W_r2; the oracle's ``backward`` is the
fp64 chain rule of its own forward (pinned to central differences).  No
gradient flows through the discrete retrieval or a hard router's choice.

Bars (derived from the arithmetic): fp32 layers accumulate every product in
fp32 over at most a few thousand terms, so each gradient is within 2e-4 of the
oracle relative to its largest entry.  bf16 layers round each gradient to bf16
where it enters an MFMA product (relative 2^-9 per operand, a few roundings in
sequence): relative L2 error <= 2e-2 and max error <= 5e-2 of the largest entry.
"""

import numpy as np
import pytest
import torch

from oracle import mka_oracle as O
from route_kv_memory_amd import inputs as I
from route_kv_memory_amd.layer import Layer, to_device

from .gpu_common import to_np
from .parity import log, oracle_kwargs, route_keep
from .test_gpu_small import SMALL

pytestmark = pytest.mark.gpu

WEIGHTS = ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")
GRADS = ("dx", "dw_q", "dw_k", "dw_v", "dw_r1", "dw_r2")


def check_grad(name, got, ref, dtype):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = max(np.abs(ref).max(), 1e-30)
    err = np.abs(got - ref).max() / scale
    rel_l2 = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    log(f"  {name}: max|ref| {scale:.3e}  max err/max|ref| {err:.2e}  rel-L2 {rel_l2:.2e}")
    if dtype == "f32":
        assert err <= 2e-4, f"{name}: {err:.2e} > 2e-4"
    else:
        assert rel_l2 <= 2e-2 and err <= 5e-2, f"{name}: rel-L2 {rel_l2:.2e}, max {err:.2e}"


def run_case(s, seed=0):
    inp = I.prefill_inputs(s)
    d_o = I.round_bf16(np.random.default_rng(seed + 100).standard_normal(
        (s.batch, s.seq, s.n_heads, s.head_dim))) if s.dtype == "bf16" else \
        np.random.default_rng(seed + 100).standard_normal(
            (s.batch, s.seq, s.n_heads, s.head_dim)).astype(np.float32)
    layer = Layer(s, inp, t_cap=s.seq, nb_cap=max(1, s.seq // s.block))
    x = to_device(inp["x"], s.dtype)
    log(f"  gpu: mka_prefill + mka_backward {s.name} ({s.route_mode}, {s.tiers})")
    out = layer.prefill(x)
    g = layer.backward(x, out, to_device(d_o, s.dtype))
    torch.cuda.synchronize()
    # hard-routing near-ties resolved to the GPU's side where that is a correct choice
    keep = route_keep(s, inp, to_np(out["lambda"]))
    ref = O.backward(inp["x"], *[inp[k] for k in WEIGHTS], d_o, keep=keep, **oracle_kwargs(s))
    return ref, out, g


CASES = [
    ("tiny_f32", "soft", "l1l2l3"), ("tiny_f32", "top2", "l1l3"), ("tiny_f32", "fixed", "l1l2"),
    ("tiny_f32", "soft", "l1"), ("small_f32_b2", "soft", "l1l2l3"),
    ("small_bf16_dh128", "soft", "l1l2l3"), ("small_bf16_dh128", "top1", "l1l3"),
    ("tiny_bf16", "soft", "l1l2l3"), ("tiny_bf16", "fixed", "l1"),
]


@pytest.mark.parametrize("base,mode,tiers", CASES)
def test_backward_matches_oracle(base, mode, tiers):
    s = SMALL[base].replace(name=f"{base}_bwd", route_mode=mode, tiers=tiers)
    ref, out, g = run_case(s)
    # the saved log-sum-exp of the forward
    fwd = ref["fwd"]
    B, N, H, dh = s.batch, s.seq, s.n_heads, s.head_dim
    qh = fwd["q"].reshape(B, N, H, dh)
    lse = np.empty((B, N, H))
    for b in range(B):
        for h in range(H):
            gg = h // (H // s.n_kv_heads)
            sc = qh[b, :, h] @ fwd["k"][b, gg].T / np.sqrt(dh)
            sc[np.triu_indices(N, 1)] = -np.inf
            mx = sc.max(axis=1, keepdims=True)
            lse[b, :, h] = (mx + np.log(np.exp(sc - mx).sum(axis=1, keepdims=True)))[:, 0]
    tol = 1e-4 if s.dtype == "f32" else 3e-2
    np.testing.assert_allclose(to_np(out["lse"]), lse, atol=tol, rtol=0)
    for k in GRADS:
        check_grad(k, to_np(g[k]), ref[k], s.dtype)


def test_backward_two_ragged_sequences_bf16():
    """Two 333-token bf16 sequences: the weight-gradient products reduce over
    666 token rows (not a multiple of the 32-row slice, rows of both
    sequences in one reduction), read K-major with the rows past the last
    token as zeros; the dq kernel runs beside the dK/dV passes."""
    s = SMALL["small_bf16_dh128"].replace(name="bwd_b2_ragged", batch=2, seed=14)
    ref, out, g = run_case(s)
    for k in GRADS:
        check_grad(k, to_np(g[k]), ref[k], s.dtype)


@pytest.mark.parametrize("base", ["small_bf16_dh128", "tiny_f32"])
def test_attention_backward_entry_matches_oracle(base):
    # mka_attn_backward alone: dq, dK, dV against the oracle's attention_backward
    # on the forward's own q, K, V (as the GPU stored them).
    from route_kv_memory_amd import mka

    s = SMALL[base]
    inp = I.prefill_inputs(s)
    layer = Layer(s, inp, t_cap=s.seq, nb_cap=max(1, s.seq // s.block))
    x = to_device(inp["x"], s.dtype)
    out = layer.prefill(x)
    r = np.random.default_rng(7)
    d_o_np = r.standard_normal((s.batch, s.seq, s.n_heads, s.head_dim))
    d_o_np = I.round_bf16(d_o_np) if s.dtype == "bf16" else d_o_np.astype(np.float32)
    d_o = to_device(d_o_np, s.dtype)
    d = layer.dims(s.seq)
    dq = torch.empty(s.batch, s.seq, s.n_heads, s.head_dim, device="cuda")
    dkv = torch.empty(s.batch, s.seq, 2, s.n_kv_heads, s.head_dim, device="cuda")
    ws = torch.empty(max(256, mka.mka_workspace_bytes(d, mka.MKA_OP_ATTN_BACKWARD)),
                     dtype=torch.uint8, device="cuda")
    mka.mka_attn_backward(d, out["q"], layer.st["k_cache"], layer.st["v_cache"], layer.t_cap,
                          out["o"], out["lse"], d_o, dq, dkv, ws, ws.numel())
    torch.cuda.synchronize()
    k = to_np(layer.st["k_cache"])[:, :, :s.seq]
    v = to_np(layer.st["v_cache"])[:, :, :s.seq]
    rq, rk, rv = O.attention_backward(to_np(out["q"]), k, v, d_o_np, s.n_kv_heads)
    g = to_np(dkv)
    check_grad("dq", to_np(dq), rq, s.dtype)
    check_grad("dk", g[:, :, 0].transpose(0, 2, 1, 3), rk, s.dtype)
    check_grad("dv", g[:, :, 1].transpose(0, 2, 1, 3), rv, s.dtype)


def test_backward_split_reduction():
    """A 1024-token bf16 layer (D = 256, 4 / 2 heads of 128): the products with
    few output tiles and a reduction over the tokens (dW_k, dW_v, dW_q, dW_r1,
    the router pre-activation, dX_fused, dx) split their reduction into 2-4
    ranges whose partials are added in order; every gradient against the oracle."""
    s = SMALL["small_bf16_dh128"].replace(name="bwd_split", seq=1024, seed=13)
    ref, out, g = run_case(s)
    for k in GRADS:
        check_grad(k, to_np(g[k]), ref[k], s.dtype)

"""GPU parity of the routing and tier variants against the oracle.

The abstract page's Table 10 compares the learned soft router with a fixed
lambda = 1/3 and hard top-2 / top-1 routing; its Table 9 removes tiers
(L1+L2, L1+L3, L1 alone).  Every variant runs through mka_prefill and
mka_decode_step with ``mka_dims.route_mode`` / ``tiers`` set, on small layers
(fp32 and bf16, ragged lengths, batch 2), and is compared with the oracle
element by element.  Outputs a variant does not write (l2 with L1 alone;
key, idx and the block codes without L3) are not compared.

Hard routing turns logits into a choice of tiers.  The oracle takes it from
its float64 logits; where those put two tiers within twice the GPU's logit
error bound of the cut (a near-tie), either side is accepted and the oracle
evaluates the side the GPU took (``route_keep``).
"""

import numpy as np
import pytest
import torch

from oracle import mka_oracle as O
from route_kv_memory_amd import inputs as I
from route_kv_memory_amd.layer import Layer, to_device

from .gpu_common import gpu_prefill, outputs_np, state_np
from .parity import check_close, check_codes, check_idx, log, oracle_kwargs, route_keep
from .test_gpu_small import SMALL

pytestmark = pytest.mark.gpu

BASES = {
    "tiny_f32": SMALL["tiny_f32"],
    "small_bf16_dh128": SMALL["small_bf16_dh128"],
    "small_f32_b2": SMALL["small_f32_b2"],
}
PREFILL_VARIANTS = [("fixed", "l1l2l3"), ("top1", "l1l2l3"), ("top2", "l1l2l3"),
                    ("soft", "l1l2"), ("soft", "l1l3"), ("soft", "l1"), ("top1", "l1l3"),
                    ("fixed", "l1l2"), ("top2", "l1")]
DECODE_VARIANTS = [("fixed", "l1l2l3"), ("top1", "l1l2l3"), ("top2", "l1l2l3"),
                   ("soft", "l1l2"), ("top2", "l1l3"), ("soft", "l1")]
WEIGHTS = ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")


def variant(base, mode, tiers):
    s = BASES[base].replace(name=f"{base}_{mode}_{tiers}", route_mode=mode, tiers=tiers)
    return s, I.prefill_inputs(s)


def oracle_for(s, inp, lam_gpu):
    """The oracle on the same inputs, hard-routing near-ties resolved to the
    GPU's side where that side is a correct choice."""
    return O.prefill(inp["x"], *[inp[k] for k in WEIGHTS], keep=route_keep(s, inp, lam_gpu),
                     **oracle_kwargs(s))


def uses_l2(s):
    return s.tiers in ("l1l2l3", "l1l2")


def uses_l3(s):
    return s.tiers in ("l1l2l3", "l1l3")


@pytest.mark.parametrize("mode,tiers", PREFILL_VARIANTS)
@pytest.mark.parametrize("base", list(BASES))
def test_variant_prefill(base, mode, tiers):
    s, inp = variant(base, mode, tiers)
    layer, out = gpu_prefill(s, inp)
    o, st = outputs_np(out), state_np(layer)
    ref = oracle_for(s, inp, o["lambda"])
    B, N = ref["lam"].shape[:2]
    check_close("q", o["q"].reshape(B, N, -1), ref["q"], s.dtype)
    check_close("lambda", o["lambda"], ref["lam"], s.dtype)
    off = [i for i, on in enumerate((True, uses_l2(s), uses_l3(s))) if not on]
    assert np.all(o["lambda"][..., off] == 0.0), "disabled tiers must have lambda = 0"
    if mode == "top1":
        assert np.all(o["lambda"].max(-1) == 1.0), "top-1 routing is one-hot"
    if s.tiers != "l1":
        check_close("l2", o["l2"], ref["l2"], "f32")
        check_close("ema_state", st["ema"], ref["l2"][:, -1], "f32")
    nb = ref["block_means"].shape[1]
    if uses_l3(s):
        check_codes("keys", o["key"], ref["keys"], ref["key_abs"], s.hash_bits)
        check_idx("idx", o["idx"], ref["keys"], ref["key_abs"], ref["block_hash"],
                  ref["block_abs"], np.arange(N), s.block, s.top_r, s.hash_bits)
        if nb:
            check_codes("block_hash", st["bhash"][:, :nb], ref["block_hash"], ref["block_abs"],
                        s.hash_bits)
    check_close("k", st["k"][:, :, :N], ref["k"], s.dtype)
    check_close("v", st["v"][:, :, :N], ref["v"], s.dtype)
    check_close("o", o["o"], ref["o"], s.dtype)


@pytest.mark.parametrize("mode,tiers", DECODE_VARIANTS)
@pytest.mark.parametrize("base,n1", [("tiny_f32", 128), ("small_bf16_dh128", 190)])
def test_variant_decode_continues_prefill(base, n1, mode, tiers):
    s, inp = variant(base, mode, tiers)
    layer = Layer(s, inp, t_cap=s.seq, nb_cap=s.seq // s.block)
    _, pre = gpu_prefill(s, inp, x=inp["x"][:, :n1], layer=layer)
    lam_pre = outputs_np(pre)["lambda"]
    xs = to_device(inp["x"], s.dtype)
    log(f"  gpu: {s.seq - n1} mka_decode_step calls ({mode}, {tiers})")
    outs = []
    for t in range(n1, s.seq):
        outs.append(outputs_np(layer.decode_step(xs[:, t:t + 1].contiguous(), t)))
    torch.cuda.synchronize()
    cat = lambda key: np.concatenate([r[key] for r in outs], axis=1)
    ref = oracle_for(s, inp, np.concatenate([lam_pre, cat("lambda")], axis=1))
    check_close("decode lambda", cat("lambda"), ref["lam"][:, n1:], s.dtype)
    check_close("decode o", cat("o"), ref["o"][:, n1:], s.dtype)
    if s.tiers != "l1":
        check_close("decode l2", cat("l2"), ref["l2"][:, n1:], "f32")
    if uses_l3(s):
        check_idx("decode idx", cat("idx"), ref["keys"][:, n1:], ref["key_abs"][:, n1:],
                  ref["block_hash"], ref["block_abs"], np.arange(n1, s.seq), s.block, s.top_r,
                  s.hash_bits)
    st = state_np(layer)
    check_close("decode k", st["k"], ref["k"], s.dtype)
    check_close("decode v", st["v"], ref["v"], s.dtype)

"""GPU parity of full MKA (three attention paths) against the oracle.

Full MKA attends each memory tier separately and mixes the outputs with the
router's lambda (reading note, method section 2); the abstract page's Table 11
contrasts its 3 paths with FastMKA's one.  mka_full_prefill and
mka_full_decode_step run on small layers (fp32, bf16 with 128-wide heads and a
ragged length, fp32 batch 2) and under routing variants; the output, lambda,
the tiers' K/V caches and the retrieval are compared with the oracle element
by element.
"""

import numpy as np
import pytest
import torch

from oracle import mka_oracle as O
from route_kv_memory_amd import inputs as I
from route_kv_memory_amd.layer import Layer, to_device

from .gpu_common import outputs_np, to_np
from .parity import check_close, check_idx, log, oracle_kwargs, route_keep
from .test_gpu_small import SMALL

pytestmark = pytest.mark.gpu

BASES = {
    "tiny_f32": SMALL["tiny_f32"],
    "small_bf16_dh128": SMALL["small_bf16_dh128"],
    "small_f32_b2": SMALL["small_f32_b2"],
}
VARIANTS = [("soft", "l1l2l3"), ("top1", "l1l3"), ("fixed", "l1l2"), ("soft", "l1")]
WEIGHTS = ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")


def setup(base, mode, tiers):
    s = BASES[base].replace(name=f"{base}_full_{mode}_{tiers}", route_mode=mode, tiers=tiers)
    return s, I.prefill_inputs(s)


def oracle_for(s, inp, lam_gpu):
    """The oracle on the same inputs, hard-routing near-ties resolved to the
    GPU's side where that side is a correct choice."""
    return O.full_prefill(inp["x"], *[inp[k] for k in WEIGHTS],
                          keep=route_keep(s, inp, lam_gpu), **oracle_kwargs(s))


def compare_caches(layer, ref, n, dtype, what="prefill"):
    for ell in range(3):
        if ref["k3"][ell] is None:
            continue
        check_close(f"{what} k tier {ell + 1}", to_np(layer.kv3["k"][ell])[:, :, :n],
                    ref["k3"][ell][:, :, :n], dtype)
        check_close(f"{what} v tier {ell + 1}", to_np(layer.kv3["v"][ell])[:, :, :n],
                    ref["v3"][ell][:, :, :n], dtype)


@pytest.mark.parametrize("mode,tiers", VARIANTS)
@pytest.mark.parametrize("base", list(BASES))
def test_full_mka_prefill(base, mode, tiers):
    s, inp = setup(base, mode, tiers)
    N = s.seq
    layer = Layer(s, inp, t_cap=N, nb_cap=max(1, N // s.block), full=True)
    log(f"  gpu: mka_full_prefill {s.name} B={s.batch} seq={N}")
    out = outputs_np(layer.full_prefill(to_device(inp["x"], s.dtype)))
    torch.cuda.synchronize()
    ref = oracle_for(s, inp, out["lambda"])
    check_close("lambda", out["lambda"], ref["lam"], s.dtype)
    if tiers in ("l1l2l3", "l1l3"):
        check_idx("idx", out["idx"], ref["keys"], ref["key_abs"], ref["block_hash"],
                  ref["block_abs"], np.arange(N), s.block, s.top_r, s.hash_bits)
    compare_caches(layer, ref, N, s.dtype)
    check_close("o", out["o"], ref["o"], s.dtype)


@pytest.mark.parametrize("mode,tiers", [("soft", "l1l2l3"), ("top1", "l1l3")])
@pytest.mark.parametrize("base,n1", [("tiny_f32", 150), ("small_bf16_dh128", 250)])
def test_full_mka_decode_continues_prefill(base, n1, mode, tiers):
    s, inp = setup(base, mode, tiers)
    layer = Layer(s, inp, t_cap=s.seq, nb_cap=s.seq // s.block, full=True)
    xs = to_device(inp["x"], s.dtype)
    lam_pre = outputs_np(layer.full_prefill(xs[:, :n1].contiguous()))["lambda"]
    log(f"  gpu: {s.seq - n1} mka_full_decode_step calls ({mode}, {tiers})")
    outs = [outputs_np(layer.full_decode_step(xs[:, t:t + 1].contiguous(), t))
            for t in range(n1, s.seq)]
    torch.cuda.synchronize()
    cat = lambda key: np.concatenate([r[key] for r in outs], axis=1)
    ref = oracle_for(s, inp, np.concatenate([lam_pre, cat("lambda")], axis=1))
    check_close("decode lambda", cat("lambda"), ref["lam"][:, n1:], s.dtype)
    check_close("decode o", cat("o"), ref["o"][:, n1:], s.dtype)
    compare_caches(layer, ref, s.seq, s.dtype, "decode")

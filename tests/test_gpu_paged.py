"""GPU checks of the paged fused KV cache and of batched decode.

The abstract page measures with a contiguous KV layout up to 32K tokens and a
paged one beyond (Table 4 caption).  With a page table in mka_state, prefill
writes and attends the cache through pages and every decode step reads and
appends through them.  A paged layer must give bit-identical outputs and
(gathered) caches to a contiguous one on the same inputs -- only addresses
differ -- and match the oracle; pages are a seeded random permutation of a
pool with spare pages.  Batched decode (B = 2..4, bf16 and fp32) is checked
against the oracle.
"""

import numpy as np
import pytest
import torch

from oracle import mka_oracle as O
from route_kv_memory_amd import inputs as I
from route_kv_memory_amd.layer import Layer, to_device

from .gpu_common import outputs_np, state_np
from .parity import check_close, check_idx, log, oracle_kwargs
from .test_gpu_small import SMALL

pytestmark = pytest.mark.gpu

WEIGHTS = ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")


def run(s, inp, n1, **layer_kw):
    """prefill(n1) then one decode step per remaining token; returns the layer
    and the decode outputs concatenated along the sequence."""
    layer = Layer(s, inp, t_cap=s.seq, nb_cap=s.seq // s.block, **layer_kw)
    xs = to_device(inp["x"], s.dtype)
    pre = outputs_np(layer.prefill(xs[:, :n1].contiguous()))
    outs = [outputs_np(layer.decode_step(xs[:, t:t + 1].contiguous(), t)) for t in range(n1, s.seq)]
    torch.cuda.synchronize()
    dec = {k: np.concatenate([r[k] for r in outs], axis=1) for k in ("o", "lambda", "idx", "l2")}
    return layer, pre, dec


CASES = [
    ("tiny_f32", 2, 64, 150),
    ("small_bf16_dh128", 2, 64, 190),
    ("small_bf16_dh128", 3, 128, 250),
]


@pytest.mark.parametrize("base,batch,page,n1", CASES)
def test_paged_cache_matches_contiguous_and_oracle(base, batch, page, n1):
    s = SMALL[base].replace(name=f"{base}_paged", batch=batch, seed=SMALL[base].seed + 20)
    inp = I.prefill_inputs(s)
    log(f"  gpu: contiguous and paged (page {page}) layers, B={batch}, prefill {n1} + decode")
    lc, pc, dc = run(s, inp, n1)
    lp, pp, dp = run(s, inp, n1, page_size=page, spare_pages=5, page_seed=7)
    assert lp.page_table is not None and lp.page_table.shape[1] * page >= s.seq
    for k in ("o", "lambda", "idx", "l2", "q"):
        np.testing.assert_array_equal(pp[k], pc[k], err_msg=f"prefill {k}")
    for k in dc:
        np.testing.assert_array_equal(dp[k], dc[k], err_msg=f"decode {k}")
    sc, sp = state_np(lc), state_np(lp)
    np.testing.assert_array_equal(sp["k"][:, :, :s.seq], sc["k"][:, :, :s.seq])
    np.testing.assert_array_equal(sp["v"][:, :, :s.seq], sc["v"][:, :, :s.seq])
    ref = O.prefill(inp["x"], *[inp[k] for k in WEIGHTS], **oracle_kwargs(s))
    check_close("paged prefill o", pp["o"], ref["o"][:, :n1], s.dtype)
    check_close("paged decode o", dp["o"], ref["o"][:, n1:], s.dtype)
    check_close("paged k", sp["k"][:, :, :s.seq], ref["k"], s.dtype)


@pytest.mark.parametrize("base,batch,n1", [("small_bf16_dh128", 4, 300), ("tiny_f32", 3, 200)])
def test_batched_decode_matches_oracle(base, batch, n1):
    s = SMALL[base].replace(name=f"{base}_b{batch}", batch=batch, seed=SMALL[base].seed + 30)
    inp = I.prefill_inputs(s)
    ref = O.prefill(inp["x"], *[inp[k] for k in WEIGHTS], **oracle_kwargs(s))
    log(f"  gpu: B={batch} prefill {n1} + {s.seq - n1} decode steps")
    layer, _, dec = run(s, inp, n1)
    check_close("batched decode o", dec["o"], ref["o"][:, n1:], s.dtype)
    check_close("batched decode lambda", dec["lambda"], ref["lam"][:, n1:], s.dtype)
    check_idx("batched decode idx", dec["idx"], ref["keys"][:, n1:], ref["key_abs"][:, n1:],
              ref["block_hash"], ref["block_abs"], np.arange(n1, s.seq), s.block, s.top_r,
              s.hash_bits)
    st = state_np(layer)
    check_close("batched decode k", st["k"], ref["k"], s.dtype)
    check_close("batched decode v", st["v"], ref["v"], s.dtype)

"""GPU check of mka_attn_decode_noalloc, the decode attention whose split
partials live in the library's device scratch instead of a caller's
workspace: two calls in a row (the second over a shorter cache, so the scratch
holds the first call's partials beyond what the second writes) must give the
same output as mka_attn_decode on the same inputs, and both the oracle's within
the bf16 bars."""

import numpy as np
import pytest
import torch

from oracle import mka_oracle as O
from route_kv_memory_amd import inputs as I
from route_kv_memory_amd import mka
from route_kv_memory_amd.layer import to_device

from .gpu_common import to_np
from .parity import check_close, log

pytestmark = pytest.mark.gpu


def test_noalloc_decode_attention_matches_workspace_entry():
    B, H, G, dh = 1, 28, 4, 128
    s = I.workload("tiny_f32").replace(dtype="bf16", n_heads=H, n_kv_heads=G, head_dim=dh,
                                       d_model=H * dh)
    d = mka.dims(s, seq=1, batch=B)
    r = np.random.default_rng(17)
    t_cap = 40000
    k = I.round_bf16(r.standard_normal((B, G, t_cap, dh)))
    v = I.round_bf16(r.standard_normal((B, G, t_cap, dh)))
    kd, vd = to_device(k, "bf16"), to_device(v, "bf16")
    for L in (40000, 777):
        q = I.round_bf16(r.standard_normal((B, 1, H, dh)))
        qd = to_device(q, "bf16")
        nbytes = mka.mka_workspace_bytes(d, mka.MKA_OP_ATTN_DECODE, L)
        assert nbytes <= mka.mka_attn_decode_noalloc_limit()
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        o_ws = torch.empty(B, 1, H, dh, dtype=torch.bfloat16, device="cuda")
        o_na = torch.full((B, 1, H, dh), float("nan"), dtype=torch.bfloat16, device="cuda")
        log(f"  gpu: mka_attn_decode and mka_attn_decode_noalloc L={L} ({nbytes} B of partials)")
        mka.mka_attn_decode(d, qd, kd, vd, t_cap, L, o_ws, ws, ws.numel())
        mka.mka_attn_decode_noalloc(d, qd, kd, vd, t_cap, L, o_na)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(o_na), to_np(o_ws))
        ref = O.attention(q, k[:, :, :L], v[:, :, :L], np.array([L - 1]), G)
        check_close(f"noalloc decode L={L}", to_np(o_na), ref, "bf16")

"""GPU parity of the route fusion and K/V projection (``mka_fuse_kv_proj``) on
bf16 layers with enough tokens (at least 1024), retrieved blocks (R >= 8) and
few enough eligible blocks (at most 256) for the matrix-core L3 path: L3[t] is the mean of the retrieved
block means (MKA reading note, method section 1), X_fused = sum_l lambda_l L_l
(section 3), [K|V] = X_fused [W_k; W_v] written into the head-major cache.
The oracle's l3_mean, fuse and kv_proj (fp64) give the reference; bars as every
bf16 output (max-abs 3e-2, mean-abs 3e-3, relative L2 1e-2).

Cases: two sequences from position 0; a call at pos0 > 0 with 128-wide heads;
exactly 256 eligible blocks (the path's limit); and retrieved indices that
name blocks outside the call's eligible range (the API allows any block below
nb_cap; they are added from the float32 means directly).  The indices are
drawn like the retrieval's: distinct eligible blocks, -1 padded.
"""

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

# (B, seq, pos0, D, G, dh, block, R, nb_cap, far)
CASES = [
    (2, 1024, 0, 256, 2, 64, 16, 16, 64, False),
    (1, 1280, 2560, 512, 2, 128, 64, 8, 64, False),
    (1, 4112, 0, 128, 1, 64, 16, 16, 260, False),
    (1, 1024, 0, 256, 2, 64, 16, 16, 80, True),
]


def draw_idx(rng, B, seq, pos0, block, R, nb_cap, far):
    idx = np.full((B, seq, R), -1, dtype=np.int32)
    n_elig = (pos0 + seq - 1) // block
    for b in range(B):
        for t in range(seq):
            ne = (pos0 + t) // block
            k = min(R, ne)
            if k:
                idx[b, t, :k] = rng.choice(ne, size=k, replace=False)
            if far and rng.random() < 0.1 and nb_cap > n_elig:
                # one slot names a block past the call's eligible range
                blk = int(rng.integers(n_elig, nb_cap))
                if blk not in idx[b, t]:
                    idx[b, t, R - 1] = blk
    return idx


@pytest.mark.parametrize("B,seq,pos0,D,G,dh,block,R,nb_cap,far", CASES)
def test_fuse_kv_proj_matches_oracle(B, seq, pos0, D, G, dh, block, R, nb_cap, far):
    rng = np.random.default_rng(seq + pos0 + D + int(far))
    x = I.round_bf16(rng.standard_normal((B, seq, D)))
    l2 = (0.07 * rng.standard_normal((B, seq, D))).astype(np.float32)
    means = (0.25 * rng.standard_normal((B, nb_cap, D))).astype(np.float32)
    z = rng.standard_normal((B, seq, 3))
    lam = (np.exp(z) / np.exp(z).sum(-1, keepdims=True)).astype(np.float32)
    w_k = I.round_bf16(rng.standard_normal((G * dh, D)) / np.sqrt(D))
    w_v = I.round_bf16(rng.standard_normal((G * dh, D)) / np.sqrt(D))
    idx = draw_idx(rng, B, seq, pos0, block, R, nb_cap, far)
    n_far = int(np.sum(idx >= (pos0 + seq - 1) // block))
    log(f"  B={B} seq={seq} pos0={pos0} D={D} block={block} R={R}: "
        f"{(pos0 + seq - 1) // block} eligible blocks, {n_far} indices past them")
    s = I.workload("tiny_f32").replace(dtype="bf16", d_model=D, n_heads=G, n_kv_heads=G,
                                       head_dim=dh, block=block, top_r=R, batch=B, seq=seq)
    d = mka.dims(s, seq=seq, batch=B)
    t_cap = pos0 + seq
    kc = torch.zeros(B, G, t_cap, dh, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    nbytes = mka.mka_workspace_bytes(d, mka.MKA_OP_FUSE_KV, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    log(f"  gpu: mka_fuse_kv_proj ({nbytes} bytes of workspace)")
    mka.mka_fuse_kv_proj(d, to_device(x, "bf16"), to_device(l2), to_device(means), nb_cap,
                         torch.from_numpy(idx).cuda(), to_device(lam), to_device(w_k, "bf16"),
                         to_device(w_v, "bf16"), kc, vc, pos0, t_cap, ws, nbytes)
    torch.cuda.synchronize()
    xf = O.fuse(lam, x, l2, O.l3_mean(means, idx))
    k_ref, v_ref = O.kv_proj(xf, w_k, w_v, G)
    check_close("k", to_np(kc)[:, :, pos0:], k_ref, "bf16")
    check_close("v", to_np(vc)[:, :, pos0:], v_ref, "bf16")
    assert np.all(to_np(kc)[:, :, :pos0] == 0.0), "rows before pos0 must be untouched"

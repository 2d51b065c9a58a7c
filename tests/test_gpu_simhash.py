"""Query codes of mka_l3_retrieve on the certified bf16 path, against the oracle;
block projections of mka_l3_block_kv at the workloads' widths.

For enough rows (B * seq >= 256, D a multiple of 32) the codes come from
bf16-split MFMA products whose signs are certified by an error bound, with
the undecided projections recomputed in float64.  The inputs here put many
projections inside that band on purpose: rows with one to three hyperplane
components removed in float64 (|v . p_j| ~ 1e-7 after rounding to float32),
zero rows, and rows scaled up and down.  Codes must equal the oracle's
float64 SimHash of the same float32 rows wherever |v . p| >= 1e-12, and the
top-R indices must equal the oracle's ranking of the GPU's codes.
"""

import numpy as np
import pytest
import torch

from oracle import mka_oracle as O
from route_kv_memory_amd import inputs as I
from route_kv_memory_amd import mka

from .parity import ambiguous_mask, check_close, log

pytestmark = pytest.mark.gpu


def adversarial_rows(rng, B, seq, D, proj):
    v = rng.normal(0.0, 0.07, (B, seq, D))
    p64 = proj.astype(np.float64)
    flat = v.reshape(-1, D)
    n = flat.shape[0]
    for i in range(0, n, 5):  # one to three components removed
        for j in rng.choice(proj.shape[0], size=1 + i % 3, replace=False):
            flat[i] -= (flat[i] @ p64[j]) / (p64[j] @ p64[j]) * p64[j]
    flat[3] = 0.0
    flat[n // 2] = 0.0
    flat[7::11] *= 1.0e3
    flat[9::13] *= 1.0e-6
    return flat.reshape(B, seq, D).astype(np.float32)


@pytest.mark.parametrize("B,seq,D,nbits,block,top_r", [
    (2, 500, 3584, 64, 128, 4),    # the Qwen2.5-7B layer's width, ragged row tiles
    (1, 300, 128, 40, 32, 2),      # narrow: half the waves have no channels; 40-bit codes
    (1, 256, 4096, 64, 256, 16),   # the Llama-3.1-8B layer's width
])
def test_certified_codes(B, seq, D, nbits, block, top_r):
    rng = np.random.default_rng(B * 1000 + D + nbits)
    proj = rng.standard_normal((nbits, D)).astype(np.float32)
    l2 = adversarial_rows(rng, B, seq, D, proj)
    nb_cap = seq // block + 1
    bhash = rng.integers(0, 2 ** 63, (B, nb_cap), dtype=np.int64).view(np.uint64)
    if nbits < 64:
        bhash &= np.uint64((1 << nbits) - 1)

    s = I.workload("tiny_f32").replace(name=f"simhash_{D}", batch=B, seq=seq, d_model=D,
                                       hash_bits=nbits, block=block, top_r=top_r)
    d = mka.dims(s)
    dev = torch.device("cuda")
    t_l2 = torch.from_numpy(l2).to(dev)
    t_proj = torch.from_numpy(proj).to(dev)
    t_bh = torch.from_numpy(bhash.view(np.int64)).to(dev)
    keys = torch.zeros((B, seq), dtype=torch.int64, device=dev)
    idx = torch.zeros((B, seq, top_r), dtype=torch.int32, device=dev)
    ws_bytes = mka.mka_workspace_bytes(d, mka.MKA_OP_RETRIEVE, 0)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    log(f"  gpu: mka_l3_retrieve B={B} seq={seq} D={D} bits={nbits} ws={ws_bytes}")
    mka.mka_l3_retrieve(d, t_l2, t_proj, t_bh, nb_cap, 0, keys, idx, ws, ws_bytes)
    torch.cuda.synchronize()
    got = keys.cpu().numpy().view(np.uint64)

    ref, pabs = O.simhash(l2, proj)
    amb = ambiguous_mask(pabs, nbits, 1e-12)
    full = np.uint64((1 << nbits) - 1) if nbits < 64 else np.uint64(0xFFFFFFFFFFFFFFFF)
    near = int(np.count_nonzero(pabs < 1e-3))
    diff = (got ^ ref) & ~amb & full
    log(f"  {np.count_nonzero(amb)} codes with |p| < 1e-12 bits; {near} projections below 1e-3; "
        f"{np.count_nonzero(diff)} codes differ")
    assert near > 100, "the inputs must put projections inside the certified band"
    assert not np.any(got & ~full), "bits above hash_bits set"
    assert np.count_nonzero(diff) == 0

    positions = np.arange(seq)
    want = np.stack([O.retrieve(got[b][None], bhash[b][None], positions, block, top_r)[0]
                     for b in range(B)])
    assert np.array_equal(idx.cpu().numpy(), want)


@pytest.mark.parametrize("B,nb_cap,first,n_blocks,D,kvw", [
    (2, 33, 0, 32, 3584, 512),     # Qwen2.5-7B layer, 2 x 4096 tokens of 128-token blocks
    (1, 300, 3, 257, 4096, 1024),  # Llama-3.1-8B layer; ragged block range across row tiles
])
def test_block_projections(B, nb_cap, first, n_blocks, D, kvw):
    """block_kv[b, blk] = m_blk [W_k; W_v]^T for the bf16 weights (split
    products on MFMA), against float64 of the same float32 means and bf16
    weights, at the float32 tolerance."""
    rng = np.random.default_rng(D + n_blocks)
    means = rng.normal(0.0, 0.09, (B, nb_cap, D)).astype(np.float32)
    wk = torch.from_numpy(rng.normal(0.0, D ** -0.5, (kvw, D)).astype(np.float32)).bfloat16()
    wv = torch.from_numpy(rng.normal(0.0, D ** -0.5, (kvw, D)).astype(np.float32)).bfloat16()
    base = "llama8b_prefill_64k" if kvw == 1024 else "qwen7b_prefill_4k"
    s = I.workload(base).replace(name=f"bkv_{D}", batch=B, d_model=D)
    assert s.n_kv_heads * s.head_dim == kvw
    d = mka.dims(s)
    dev = torch.device("cuda")
    out = torch.full((B, nb_cap, 2 * kvw), 7.0, dtype=torch.float32, device=dev)
    log(f"  gpu: mka_l3_block_kv B={B} blocks {first}..{first + n_blocks} D={D} kvw={kvw}")
    mka.mka_l3_block_kv(d, torch.from_numpy(means).to(dev), nb_cap, first, n_blocks,
                        wk.to(dev), wv.to(dev), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    w = torch.cat([wk, wv]).float().numpy().astype(np.float64)
    want = means[:, first:first + n_blocks].astype(np.float64) @ w.T
    check_close("block_kv", got[:, first:first + n_blocks], want, "f32")
    # rows outside the range are left alone
    assert np.all(got[:, :first] == 7.0) and np.all(got[:, first + n_blocks:] == 7.0)

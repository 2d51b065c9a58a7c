"""Comparison helpers shared by the GPU parity tests (the HIP path vs the oracle).

Tolerances: fp32 layers max-abs 1e-4 and relative L2 error 1e-5; bf16
layers max-abs 3e-2, mean-abs 3e-3 and relative L2 error 1e-2, on unit-scale
inputs.  The relative L2 bar keeps the absolute bars meaningful where outputs
are small (a softmax-weighted mean over many keys).  Integer results (block
indices) are compared exactly; SimHash bits whose oracle projection |p| is
below 1e-6 are treated as undetermined (either value accepted) and a ranking
is accepted if it matches the oracle's ranking for some assignment of those
bits.  Hard routing is treated the same way: where the oracle's float64
logits put two tiers within twice the logit error bound of the cut, either
side of the cut is accepted and the oracle evaluates the side the GPU took.
"""

from __future__ import annotations

import itertools
import sys

import numpy as np

from oracle import mka_oracle as O

AMBIG = 1e-6
MAX_AMBIG_BITS = 10

TOL = {"f32": dict(max_abs=1e-4, mean_abs=None, rel_l2=1e-5),
       "bf16": dict(max_abs=3e-2, mean_abs=3e-3, rel_l2=1e-2)}

# Bound on |z_gpu - z|, the difference between the GPU's router logits and
# the oracle's float64 ones.  bf16 layers store q in bf16 (relative rounding
# 2^-9 per entry): over the D-long first layer and the r-long second layer of
# unit-scale data that moves a logit by ~1e-3 (rms), so 2e-2 is a bound with
# a wide margin; fp32 layers accumulate in fp32 (~1e-6).
ROUTE_TIE = {"bf16": 2e-2, "f32": 1e-5}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_kwargs(s):
    """Hyper-parameters as the GPU receives them (the decay as float32)."""
    return dict(n_heads=s.n_heads, n_kv_heads=s.n_kv_heads,
                ema_decay=float(np.float32(s.ema_decay)), block=s.block, top_r=s.top_r,
                route_mode=s.route_mode, tiers=s.tiers)


def check_close(name, got, ref, dtype, max_abs=None, mean_abs=None, rel_l2=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    tol = TOL[dtype]
    ma = tol["max_abs"] if max_abs is None else max_abs
    mn = tol["mean_abs"] if mean_abs is None else mean_abs
    rel_l2 = tol["rel_l2"] if rel_l2 is None else rel_l2
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    log(f"  {name}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} rel_l2={rel:.3e}")
    assert err.max() <= ma, f"{name}: max abs err {err.max():.3e} > {ma:.1e}"
    if mn is not None:
        assert err.mean() <= mn, f"{name}: mean abs err {err.mean():.3e} > {mn:.1e}"
    if rel_l2 is not None:
        assert rel <= rel_l2, f"{name}: relative L2 error {rel:.3e} > {rel_l2:.1e}"
    return dict(max_abs=float(err.max()), mean_abs=float(err.mean()), rel_l2=rel)


def ambiguous_mask(absp, nbits, thresh=AMBIG):
    """uint64 masks of the bits whose |projection| < thresh."""
    absp = np.asarray(absp)
    w = np.left_shift(np.uint64(1), np.arange(nbits, dtype=np.uint64))
    return ((absp < thresh).astype(np.uint64) * w).sum(axis=-1, dtype=np.uint64)


def check_codes(name, got, ref, ref_abs, nbits):
    """Bitwise equality of SimHash codes outside the undetermined bits."""
    got = np.asarray(got).view(np.uint64) if np.asarray(got).dtype != np.uint64 else np.asarray(got)
    ref = np.asarray(ref, dtype=np.uint64)
    amb = ambiguous_mask(ref_abs, nbits)
    full = np.uint64((1 << nbits) - 1) if nbits < 64 else np.uint64(0xFFFFFFFFFFFFFFFF)
    diff = (got ^ ref) & ~amb & full
    bad = np.count_nonzero(diff)
    log(f"  {name}: {got.size} codes, {int(np.count_nonzero(amb))} with undetermined bits, "
        f"{bad} mismatching")
    assert bad == 0, f"{name}: {bad} codes differ outside undetermined bits"
    assert not np.any(got & ~full), f"{name}: bits above hash_bits set"


def check_idx(name, got, keys, key_abs, bhash, babs, positions, block, top_r, nbits):
    """Exact block indices, allowing any assignment of undetermined bits."""
    got = np.asarray(got)
    positions = np.asarray(positions)
    B, n, R = got.shape
    kamb = ambiguous_mask(key_abs, nbits)
    bamb = ambiguous_mask(babs, nbits)
    skipped = relaxed = 0
    for b in range(B):
        ref = O.retrieve(keys[b][None], bhash[b][None], positions, block, top_r)[0]
        for i in range(n):
            if np.array_equal(got[b, i], ref[i]):
                continue
            t = int(positions[i])
            ne = t // block
            bits = [("k", 0, j) for j in range(nbits) if (int(kamb[b, i]) >> j) & 1]
            for blk in range(ne):
                bits += [("b", blk, j) for j in range(nbits) if (int(bamb[b, blk]) >> j) & 1]
            if not bits:
                raise AssertionError(f"{name}: row b={b} t={t}: gpu {got[b, i]} != oracle {ref[i]}")
            if len(bits) > MAX_AMBIG_BITS:
                skipped += 1
                continue
            ok = False
            for assign in itertools.product((0, 1), repeat=len(bits)):
                k = int(keys[b, i])
                hb = bhash[b, :ne].copy()
                for (kind, blk, j), v in zip(bits, assign):
                    if kind == "k":
                        k = (k & ~(1 << j)) | (v << j)
                    else:
                        hb[blk] = np.uint64((int(hb[blk]) & ~(1 << j)) | (v << j))
                alt = O.retrieve(np.array([[k]], dtype=np.uint64), hb[None], np.array([t]),
                                 block, top_r)[0, 0]
                if np.array_equal(alt, got[b, i]):
                    ok = True
                    break
            assert ok, f"{name}: row b={b} t={t}: gpu {got[b, i]} matches no assignment"
            relaxed += 1
    log(f"  {name}: {B * n} rows exact ({relaxed} via undetermined bits, {skipped} skipped)")


def check_idx_conditional(name, got_idx, got_keys, gpu_l2, gpu_means, gpu_bhash, proj, positions,
                          block, top_r, nbits):
    """Retrieval re-ranked by the oracle from the GPU's own L2 and block means.

    Isolates hashing and top-R selection from the rounding of the scan: with
    identical float32 inputs the codes are determined up to |p| ~ 1e-12."""
    keys, kabs = O.simhash(gpu_l2, proj)
    bh, babs = O.simhash(gpu_means, proj)
    amb_k = ambiguous_mask(kabs, nbits, 1e-12)
    amb_b = ambiguous_mask(babs, nbits, 1e-12)
    full = np.uint64((1 << nbits) - 1) if nbits < 64 else np.uint64(0xFFFFFFFFFFFFFFFF)
    gk = np.asarray(got_keys).view(np.uint64)
    gb = np.asarray(gpu_bhash).view(np.uint64)
    assert not np.any((gk ^ keys) & ~amb_k & full), f"{name}: keys differ given the GPU's L2"
    assert not np.any((gb ^ bh) & ~amb_b & full), f"{name}: block codes differ given the GPU's means"
    ref = np.stack([O.retrieve(gk[b][None], gb[b][None], positions, block, top_r)[0]
                    for b in range(gk.shape[0])])
    bad = np.argwhere(np.any(ref != np.asarray(got_idx), axis=-1))
    assert len(bad) == 0, f"{name}: {len(bad)} rows differ from the oracle ranking of the GPU's codes"
    log(f"  {name}: conditional retrieval exact on {ref.shape[0] * ref.shape[1]} rows")


def route_keep(s, inp, lam_gpu, x=None):
    """Each token's kept tiers for the oracle under hard routing, or None.

    The oracle's choice is taken from its float64 logits z.  The GPU's logits
    differ from z by at most e = ROUTE_TIE[dtype], so where a kept and a
    dropped enabled tier lie within 2e of each other either side of the cut
    is a correct choice (a near-tie, as an undetermined SimHash bit).  At
    such tokens the GPU's choice (the non-zero entries of its lambda) is
    accepted if it is consistent with z within 2e, and returned for the
    oracle to evaluate; everywhere else the GPU must match the float64
    choice exactly (the later lambda comparison checks that).  ``x``: the
    hiddens the GPU routed (default inp["x"]).
    """
    k = {"top1": 1, "top2": 2}.get(s.route_mode)
    on = [i for i, e in enumerate(O.TIER_SETS[s.tiers]) if e]
    if k is None or k >= len(on):
        return None
    x = inp["x"] if x is None else x
    z = O.router_logits(O.q_proj(x, inp["w_q"]), inp["w_r1"], inp["w_r2"])
    keep = O.route_choice(z, s.route_mode, s.tiers)
    zon = z[..., on]
    zs = -np.sort(-zon, axis=-1)
    tie = (zs[..., k - 1] - zs[..., k]) < 2.0 * ROUTE_TIE[s.dtype]
    got = np.asarray(lam_gpu) > 0.0
    out = keep.copy()
    flipped = 0
    for idx in zip(*np.nonzero(tie)):
        g = got[idx]
        assert g.sum() == k and all(g[i] == 0 for i in range(3) if i not in on), \
            f"token {idx}: GPU keeps tiers {np.nonzero(g)[0]} under {s.route_mode}/{s.tiers}"
        kept_min = min(z[idx][i] for i in range(3) if g[i])
        dropped_max = max((z[idx][i] for i in on if not g[i]), default=-np.inf)
        assert kept_min >= dropped_max - 2.0 * ROUTE_TIE[s.dtype], \
            f"token {idx}: GPU choice {np.nonzero(g)[0]} is not within the tie bound of z {z[idx]}"
        flipped += int(not np.array_equal(g, keep[idx]))
        out[idx] = g
    log(f"  route_keep: {int(tie.sum())} near-tie tokens of {tie.size} "
        f"(margin < {2.0 * ROUTE_TIE[s.dtype]:.0e}), {flipped} took the other side")
    return out

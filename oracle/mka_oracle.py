"""CPU oracle of the FastMKA layer forward (prefill and decode).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
HIP library never calls it, and it shares no code with the HIP library: the
two meet only in the seeded input arrays of ``route_kv_memory_amd.inputs``.

Plain NumPy in float64 throughout.  Inputs are the exact values the GPU
receives (bf16 workloads: already rounded to bf16), widened to float64.
Each function is the definition written out, in the order the pages give it;
library primitives (matmul, erf, sort) are the only helpers.

Sources (the two pages about the method):
  * "MKA reading note" -- Paper-Notes page "MKA: Memory-Keyed Attention for
    Efficient Long-Context Reasoning" (method sections 1-4).
  * "MKA abstract page" -- the paper's landing page of the same title
    (abstract, Tables 1-11 and their captions).

Where the pages leave a step open, the reading taken is stated at the
function.  The fixed readings: L2 is an exponential moving average with a
stated decay; L3 is SimHash of past complete-block means, keyed by the
SimHash of L2[t], keeping the top-R blocks by Hamming distance with ties
broken towards the most recent block.

Parity pins: every function here is pinned by a test in
``tests/test_oracle_pins.py`` (closed forms, special cases, brute force on
tiny inputs, invariants).  The composite ``prefill``/``decode`` with general
router weights and non-empty L3 has no end-to-end worked example on the
pages; it rests on its pinned parts plus the special cases (one-hot router
equals causal GQA attention, decode continues prefill, causality) -- beyond
those it is "parity unpinned".  The routing variants (``route_weights``) are
pinned to scipy's softmax over the enabled tiers, a brute force over tier
subsets, hand-made ties, torch's attention for L1 alone, and invariances
(fixed routing ignores the router weights; without L3 the hash index does
not matter).  Full MKA (``full_prefill``, ``full_decode_step``) is pinned
path by path to torch's attention over each tier's keys and values, to
FastMKA and plain GQA where the tiers coincide, and by decode continuing
prefill.  The backward (``backward``) is pinned to central differences of
this module's own forward (every parameter tensor, three routing variants),
its attention part to torch's autograd of its scaled-dot-product attention,
the EMA and L3 steps by adjoint identities, GELU' to torch's autograd.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "q_proj", "gelu", "router", "router_logits", "route_choice", "route_weights", "ROUTE_MODES",
    "TIER_SETS",
    "ema", "block_means", "simhash", "retrieve",
    "l3_mean", "fuse", "kv_proj", "attention", "attention_online", "prefill",
    "DecodeState", "decode_init", "decode_init_from_prefill", "decode_step",
    "full_prefill", "FullDecodeState", "full_decode_init_from_prefill", "full_decode_step",
    "gelu_grad", "attention_backward", "ema_adjoint", "l3_adjoint", "backward",
]

_SQRT2 = math.sqrt(2.0)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Router: lambda = softmax(MLP(q)), one 3-vector per token and layer.
# MKA reading note, section 2 (dynamic routing gate).
# --------------------------------------------------------------------------

def q_proj(x, w_q):
    """Q = X W_q (no bias, no rotary encoding).  ``w_q`` is stored [out, in].

    Reading: the "q" fed to the router is this same query projection of the
    token hidden (the note introduces q per token and uses its per-head slices
    q_h as attention queries); it cannot be taken from the fused input, since
    the router output is what forms the fused input.
    """
    return _f64(x) @ _f64(w_q).T


def gelu(z):
    """Exact GELU, z * Phi(z) = z/2 * (1 + erf(z / sqrt 2))."""
    z = _f64(z)
    return 0.5 * z * (1.0 + _erf(z / _SQRT2))


def _softmax(z):
    z = _f64(z)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# Routing variants of the abstract page's ablations: Table 10 compares the
# learned soft router with a fixed lambda = 1/3 and hard top-2 / top-1
# routing; Table 9 removes tiers (L1+L2, L1+L3, L1 alone, the last being
# plain multi-head attention).
ROUTE_MODES = ("soft", "fixed", "top1", "top2")
TIER_SETS = {
    "l1l2l3": (True, True, True),
    "l1l2": (True, True, False),
    "l1l3": (True, False, True),
    "l1": (True, False, False),
}


def router_logits(q, w_r1, w_r2):
    """z = GELU(q W_r1) W_r2, the three tier logits before the softmax.

    MKA reading note, section 2: a learned MLP of the query gives the gate.
    Reading: a two-layer MLP with an exact GELU between the layers and no
    biases.  Output [..., 3]; tier 0 = L1, 1 = L2, 2 = L3.
    """
    return gelu(_f64(q) @ _f64(w_r1).T) @ _f64(w_r2).T


def route_choice(z, mode="soft", tiers="l1l2l3"):
    """The kept tiers [..., 3] (bool) of a routing variant, from the logits z.

    soft keeps every enabled tier; top1 / top2 keep the k enabled tiers with
    the largest logits, ties going to the lower tier index (abstract page,
    Table 10's hard routing); fixed keeps every enabled tier.
    """
    z = _f64(z)
    en = TIER_SETS[tiers]
    on = [i for i in range(3) if en[i]]
    k = {"soft": 3, "fixed": 3, "top1": 1, "top2": 2}[mode]
    keep = np.zeros(z.shape, dtype=bool)
    for i in on:
        # rank of tier i among the enabled tiers: how many beat it
        rank = np.zeros(z.shape[:-1], dtype=np.int64)
        for j in on:
            if j != i:
                beats = (z[..., j] > z[..., i]) | ((z[..., j] == z[..., i]) & (j < i))
                rank += beats.astype(np.int64)
        keep[..., i] = rank < k
    return keep


def route_weights(z, mode="soft", tiers="l1l2l3", keep=None):
    """lambda from the logits z [..., 3] under a routing variant.

    ``tiers`` names the enabled tiers (L1 is always one); the others get
    lambda = 0.  ``mode``:
      soft  -- softmax of z over the enabled tiers (with all three: the
               learned router of the reading note, section 2);
      fixed -- 1 / (number of enabled tiers) on each, z unused (abstract
               page, Table 10: lambda = 1/3 with all three);
      top1, top2 -- the k enabled tiers with the largest logits
               (``route_choice``) and a softmax over those k alone (Table
               10's hard routing).  Readings: the kept weights are
               renormalised, as a softmax restricted to the kept tiers; top-1
               is therefore one-hot, and top-k with k >= the enabled count is
               soft.
    ``keep`` [..., 3] (bool), when given, names the kept tiers instead of the
    ranking of z: the weights of another choice of tiers (a comparison that
    accepts either side of an exact tie evaluates both this way).
    """
    z = _f64(z)
    en = TIER_SETS[tiers]
    on = [i for i in range(3) if en[i]]
    lam = np.zeros(z.shape)
    if mode == "fixed":
        for i in on:
            lam[..., i] = 1.0 / len(on)
        return lam
    keep = route_choice(z, mode, tiers) if keep is None else np.asarray(keep, dtype=bool)
    zk = np.where(keep, z, -np.inf)
    e = np.where(keep, np.exp(zk - zk.max(axis=-1, keepdims=True)), 0.0)
    return e / e.sum(axis=-1, keepdims=True)


def router(q, w_r1, w_r2, mode="soft", tiers="l1l2l3", keep=None):
    """lambda = softmax(GELU(q W_r1) W_r2) over the three memory tiers.

    MKA reading note, section 2: a learned MLP of the query followed by a
    softmax gives lambda in R^{B x S x 3}, per token and per layer.  Other
    ``mode`` / ``tiers`` values give the ablation variants (``route_weights``;
    ``keep`` as there).  Output [..., 3]; tier 0 = L1, 1 = L2, 2 = L3.
    """
    z = router_logits(q, w_r1, w_r2)
    if mode == "soft" and tiers == "l1l2l3":
        return _softmax(z)
    return route_weights(z, mode, tiers, keep=keep)


# --------------------------------------------------------------------------
# L2 session memory: causal summary of the prefix.
# MKA reading note, section 1 (three-tier memory; M2[t] = Summary(X[:, 1:t])).
# --------------------------------------------------------------------------

def ema(x, beta, state=None):
    """Exponential moving average along the sequence axis.

    s_{-1} = state (zeros if None); s_t = beta * s_{t-1} + (1 - beta) * x_t;
    L2[t] = s_t.  The note allows "a low-rank summary or an EMA"; the EMA is
    the reading taken.  The prefix includes token t itself (the note's
    X[:, 1:t] in 1-based indexing), which uses no future token.

    x: [B, N, D].  Returns (L2 [B, N, D], final state [B, D]).
    """
    x = _f64(x)
    B, N, D = x.shape
    s = np.zeros((B, D)) if state is None else _f64(state).copy()
    out = np.empty((B, N, D))
    for t in range(N):
        s = beta * s + (1.0 - beta) * x[:, t]
        out[:, t] = s
    return out, s


# --------------------------------------------------------------------------
# L3 long-term memory: hashed retrieval of R past blocks.
# MKA reading note, section 1 (vectorised hash index over past blocks,
# recalling R << T blocks) and section 4 (blockwise evaluation);
# MKA abstract page, Table 8 caption (R = 8 retrieved chunks per query).
# --------------------------------------------------------------------------

def block_means(x, block):
    """Mean of the token hiddens over every complete block of ``block`` tokens.

    Reading: blocks are fixed-size runs of tokens (the pages' content-defined
    chunking is not specified), and a block is summarised by the mean of its
    raw token hiddens, so that L3 lives in d_model space like L1 and L2.
    x: [B, N, D] -> [B, N // block, D].
    """
    x = _f64(x)
    B, N, D = x.shape
    nb = N // block
    return x[:, : nb * block].reshape(B, nb, block, D).mean(axis=2)


def simhash(v, proj):
    """SimHash code of each row of ``v`` against the hyperplanes in ``proj``.

    p = v . proj_j for each hyperplane j; bit j of the code is 1 iff p_j > 0
    (p_j = 0 gives 0).  proj: [nbits, D] with nbits <= 64.
    Returns (codes uint64 [...], |p| [..., nbits]).
    """
    p = _f64(v) @ _f64(proj).T
    nbits = p.shape[-1]
    if nbits > 64:
        raise ValueError("at most 64 hash bits")
    bits = (p > 0).astype(np.uint64)
    weights = np.left_shift(np.uint64(1), np.arange(nbits, dtype=np.uint64))
    codes = (bits * weights).sum(axis=-1, dtype=np.uint64)
    return codes, np.abs(p)


def _popcount64(a):
    a = np.asarray(a, dtype=np.uint64)
    return np.bitwise_count(a).astype(np.int64)


def retrieve(keys, block_hash, positions, block, top_r):
    """Top-R past blocks for each token, by Hamming distance of SimHash codes.

    For the token at position t, the eligible blocks are b < floor(t / block):
    the complete blocks strictly before t's own block (t's own block is the
    local window that L1 covers).  They are ranked by (popcount(key_t xor
    hash_b) ascending, b descending) -- equal distances go to the most recent
    block -- and the first min(R, #eligible) are kept, in rank order; the rest
    of the R slots hold -1.

    keys: [B, n] uint64 for tokens at ``positions`` [n]; block_hash [B, nb].
    Returns idx int32 [B, n, R].
    """
    keys = np.asarray(keys, dtype=np.uint64)
    block_hash = np.asarray(block_hash, dtype=np.uint64)
    positions = np.asarray(positions, dtype=np.int64)
    B, n = keys.shape
    nb = block_hash.shape[1]
    out = np.full((B, n, top_r), -1, dtype=np.int32)
    for b in range(B):
        for i in range(n):
            ne = int(positions[i]) // block
            if ne > nb:
                raise ValueError("block index is missing eligible blocks")
            if ne == 0:
                continue
            cand = np.arange(ne, dtype=np.int64)
            dist = _popcount64(np.bitwise_xor(block_hash[b, :ne], keys[b, i]))
            order = np.lexsort((-cand, dist))  # primary: dist asc; then b desc
            sel = cand[order][:top_r]
            out[b, i, : len(sel)] = sel
    return out


def l3_mean(means, idx):
    """L3[t] = mean of the retrieved block means (zero when none is eligible).

    means [B, nb, D]; idx [B, n, R] with -1 padding -> [B, n, D].
    """
    means = _f64(means)
    B, n, R = idx.shape
    out = np.zeros((B, n, means.shape[2]))
    for b in range(B):
        for i in range(n):
            sel = idx[b, i][idx[b, i] >= 0]
            if len(sel):
                out[b, i] = means[b, sel].mean(axis=0)
    return out


# --------------------------------------------------------------------------
# FastMKA: fuse the tiers before attention, project K and V from the fusion.
# MKA reading note, section 3 (X_fused = sum_l lambda_l * L_l; K, V =
# X_fused W_k, X_fused W_v; one causal attention; the fused K/V is cached);
# MKA abstract page, abstract ("broadcast-routed": lambda is a per-token
# scalar per tier, broadcast over d_model).
# --------------------------------------------------------------------------

def fuse(lam, l1, l2, l3):
    """X_fused = lambda_1 L1 + lambda_2 L2 + lambda_3 L3, lambda broadcast over D.

    L1 is the token's own hidden x_t.
    """
    lam = _f64(lam)
    return lam[..., 0:1] * _f64(l1) + lam[..., 1:2] * _f64(l2) + lam[..., 2:3] * _f64(l3)


def kv_proj(x_fused, w_k, w_v, n_kv_heads):
    """K = X_fused W_k, V = X_fused W_v, returned head-major [B, G, n, dh]."""
    xf = _f64(x_fused)
    B, n, _ = xf.shape
    k = xf @ _f64(w_k).T
    v = xf @ _f64(w_v).T
    dh = k.shape[-1] // n_kv_heads
    k = k.reshape(B, n, n_kv_heads, dh).transpose(0, 2, 1, 3)
    v = v.reshape(B, n, n_kv_heads, dh).transpose(0, 2, 1, 3)
    return k, v


# --------------------------------------------------------------------------
# One standard causal attention over the fused K/V.
# MKA reading note, section 3 (single attention path) and section 4 (online
# max-shift); models are GQA (reading note, experimental setup).
# --------------------------------------------------------------------------

def _group_of(h, n_heads, n_kv_heads):
    # Contiguous groups: query heads [g*H/G, (g+1)*H/G) share KV head g.
    return h // (n_heads // n_kv_heads)


def attention(q, k, v, positions, n_kv_heads):
    """Causal GQA attention, explicit scores and a two-pass softmax.

    O[t, h] = sum_{j <= t} softmax_j(q_{t,h} . k_{j,g(h)} / sqrt(dh)) v_{j,g(h)}.
    The 1/sqrt(dh) scale is that of standard attention (the note's formula
    omits it); the mask keeps j <= t, the token itself included.

    q: [B, n, H, dh] for query tokens at ``positions`` [n];
    k, v: [B, G, T, dh] with T > max(positions).  Returns [B, n, H, dh].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, n, H, dh = q.shape
    positions = np.asarray(positions, dtype=np.int64)
    T = int(positions.max()) + 1
    scale = 1.0 / math.sqrt(dh)
    out = np.empty((B, n, H, dh))
    future = np.arange(T)[None, :] > positions[:, None]  # [n, T]
    for b in range(B):
        for h in range(H):
            g = _group_of(h, H, n_kv_heads)
            s = (q[b, :, h] @ k[b, g, :T].T) * scale
            s[future] = -np.inf
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            out[b, :, h] = (p @ v[b, g, :T]) / p.sum(axis=1, keepdims=True)
    return out


def attention_online(q, k, v, positions, n_kv_heads, tile=64):
    """The same attention evaluated key tile by key tile with the online max-shift.

    MKA reading note, section 4: the running maximum mu is updated tile by
    tile, and the running numerator and denominator are rescaled by
    exp(mu_old - mu_new) whenever it grows.  Used to cross-check
    ``attention``; shares none of its code.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, n, H, dh = q.shape
    positions = np.asarray(positions, dtype=np.int64)
    scale = 1.0 / math.sqrt(dh)
    out = np.empty((B, n, H, dh))
    for b in range(B):
        for h in range(H):
            g = _group_of(h, H, n_kv_heads)
            for i in range(n):
                t = int(positions[i])
                mu = -np.inf
                den = 0.0
                num = np.zeros(dh)
                for j0 in range(0, t + 1, tile):
                    j1 = min(j0 + tile, t + 1)
                    s = (k[b, g, j0:j1] @ q[b, i, h]) * scale
                    mu_new = max(mu, float(s.max()))
                    corr = math.exp(mu - mu_new) if mu != -np.inf else 0.0
                    p = np.exp(s - mu_new)
                    den = den * corr + p.sum()
                    num = num * corr + p @ v[b, g, j0:j1]
                    mu = mu_new
                out[b, i, h] = num / den
    return out


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

def prefill(x, w_q, w_k, w_v, w_r1, w_r2, proj, *, n_heads, n_kv_heads, ema_decay,
            block, top_r, rows=None, lam_override=None, route_mode="soft", tiers="l1l2l3",
            keep=None):
    """FastMKA layer forward over a whole sequence (every step, in page order).

    Returns a dict with q [B,N,H*dh], lam [B,N,3], l2 [B,N,D], block_means
    [B,nb,D], block_hash [B,nb], block_abs [B,nb,nbits], keys [B,N],
    key_abs [B,N,nbits], idx [B,N,R], l3 [B,N,D], x_fused [B,N,D],
    k, v [B,G,N,dh], rows [n] and o [B,n,H,dh] (attention only at ``rows``;
    every row otherwise).  ``lam_override`` [B,N,3] replaces the router output;
    ``route_mode`` and ``tiers`` select a routing variant (``route_weights``;
    ``keep`` [B,N,3], when given, names each token's kept tiers).
    Every tier is computed whatever the variant; a disabled tier enters the
    fusion with lambda = 0.
    """
    x = _f64(x)
    B, N, D = x.shape
    q = q_proj(x, w_q)
    lam = (router(q, w_r1, w_r2, route_mode, tiers, keep) if lam_override is None
           else _f64(lam_override))
    l2, _ = ema(x, ema_decay)
    means = block_means(x, block)
    bhash, babs = simhash(means, proj)
    keys, kabs = simhash(l2, proj)
    idx = retrieve(keys, bhash, np.arange(N), block, top_r)
    l3 = l3_mean(means, idx)
    xf = fuse(lam, x, l2, l3)
    k, v = kv_proj(xf, w_k, w_v, n_kv_heads)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    dh = q.shape[-1] // n_heads
    q_rows = q[:, rows].reshape(B, len(rows), n_heads, dh)
    o = attention(q_rows, k, v, rows, n_kv_heads)
    return dict(q=q, lam=lam, l2=l2, block_means=means, block_hash=bhash, block_abs=babs,
                keys=keys, key_abs=kabs, idx=idx, l3=l3, x_fused=xf, k=k, v=v, rows=rows, o=o)


class DecodeState:
    """Carried decode state: fused KV cache, EMA state, partial block sum,
    block means and their hashes, and the position of the next token."""

    def __init__(self, k, v, ema_state, block_acc, means, pos):
        self.k = _f64(k).copy()
        self.v = _f64(v).copy()
        self.ema_state = _f64(ema_state).copy()
        self.block_acc = _f64(block_acc).copy()
        self.means = _f64(means).copy()
        self.pos = int(pos)
        self.hash = None
        self.hash_abs = None


def decode_init(k_cache, v_cache, ema_state, block_acc, means, proj, *, t_cap):
    """State for decoding after ``k_cache.shape[2]`` cached tokens.

    Room for ``t_cap`` rows is reserved in the cache.  Block hashes are
    computed here from the given block means.
    """
    k_cache, v_cache = _f64(k_cache), _f64(v_cache)
    B, G, T0, dh = k_cache.shape
    k = np.zeros((B, G, t_cap, dh))
    v = np.zeros((B, G, t_cap, dh))
    k[:, :, :T0] = k_cache
    v[:, :, :T0] = v_cache
    st = DecodeState(k, v, ema_state, block_acc, means, T0)
    st.hash, st.hash_abs = simhash(st.means, proj)
    return st


def decode_init_from_prefill(x, ref, proj, *, block, t_cap):
    """State after a prefill (``ref`` = the dict ``prefill`` returned)."""
    x = _f64(x)
    B, N, D = x.shape
    nb = N // block
    acc = x[:, nb * block:].sum(axis=1)
    return decode_init(ref["k"], ref["v"], ref["l2"][:, -1], acc, ref["block_means"], proj,
                       t_cap=t_cap)


def decode_step(st, x_t, w_q, w_k, w_v, w_r1, w_r2, proj, *, n_heads, n_kv_heads, ema_decay,
                block, top_r, attend=True, route_mode="soft", tiers="l1l2l3", keep=None):
    """One decode step at position t = st.pos for the token hiddens x_t [B, D].

    The same definitions as ``prefill`` applied to one token with the carried
    state; the fused K/V row is appended to the cache.  When token t closes a
    block ((t + 1) mod block == 0) the block mean is finalised, hashed and
    appended to the index; it becomes eligible from the next block on.
    Returns a dict with q, lam, l2, key, key_abs, idx, k_row, v_row and o
    ([B, H, dh], or None when ``attend`` is False).
    """
    x_t = _f64(x_t)
    B, D = x_t.shape
    t = st.pos
    q = q_proj(x_t, w_q)
    lam = router(q, w_r1, w_r2, route_mode, tiers, keep)
    l2_seq, st.ema_state = ema(x_t[:, None, :], ema_decay, st.ema_state)
    l2 = l2_seq[:, 0]
    st.block_acc = st.block_acc + x_t
    key, kabs = simhash(l2, proj)
    idx = retrieve(key[:, None], st.hash, np.array([t]), block, top_r)
    l3 = l3_mean(st.means, idx)[:, 0]
    xf = fuse(lam, x_t, l2, l3)
    k_row, v_row = kv_proj(xf[:, None, :], w_k, w_v, n_kv_heads)
    st.k[:, :, t] = k_row[:, :, 0]
    st.v[:, :, t] = v_row[:, :, 0]
    o = None
    if attend:
        dh = q.shape[-1] // n_heads
        o = attention(q.reshape(B, 1, n_heads, dh), st.k, st.v, np.array([t]), n_kv_heads)[:, 0]
    if (t + 1) % block == 0:
        m = st.block_acc / block
        h, habs = simhash(m, proj)
        st.means = np.concatenate([st.means, m[:, None]], axis=1)
        st.hash = np.concatenate([st.hash, h[:, None]], axis=1)
        st.hash_abs = np.concatenate([st.hash_abs, habs[:, None]], axis=1)
        st.block_acc = np.zeros_like(st.block_acc)
    st.pos = t + 1
    return dict(q=q, lam=lam, l2=l2, key=key, key_abs=kabs, idx=idx[:, 0], l3=l3,
                x_fused=xf, k_row=k_row[:, :, 0], v_row=v_row[:, :, 0], o=o)


# --------------------------------------------------------------------------
# Full MKA: three attention paths, mixed after attention.
# MKA reading note, section 2 (O_h = sum_l lambda_l * a_l, a_l = softmax(q_h
# k_l^T) v_l, the attention output of memory tier l); section 3 contrasts it
# with FastMKA, which fuses the tiers before one attention; the abstract
# page's Table 11 counts 3 attention paths and 9 launches for it.
#
# Reading: tier l's keys and values at position j are L_l[j] W_k and
# L_l[j] W_v, with the same tiers L1 = x, L2 = EMA, L3 = mean of the
# retrieved block means as in FastMKA and the same W_k, W_v; each path is one
# causal attention over its own cache; lambda (per token and tier) is
# broadcast over heads and head dimensions.  A disabled tier (``tiers``) has
# lambda = 0 and its path is left out.
# --------------------------------------------------------------------------

def full_prefill(x, w_q, w_k, w_v, w_r1, w_r2, proj, *, n_heads, n_kv_heads, ema_decay,
                 block, top_r, rows=None, route_mode="soft", tiers="l1l2l3", keep=None):
    """Full MKA forward over a whole sequence.

    Returns a dict with q, lam, l2, block_means, block_hash, block_abs, keys,
    key_abs, idx, l3 (as ``prefill``), k3 and v3 (lists of the three tiers'
    [B,G,N,dh] caches; None for a disabled tier), a3 (the three paths'
    attention outputs at ``rows``, [B,n,H,dh]; None when disabled), rows and
    o = sum_l lambda_l a_l [B,n,H,dh].
    """
    x = _f64(x)
    B, N, D = x.shape
    q = q_proj(x, w_q)
    lam = router(q, w_r1, w_r2, route_mode, tiers, keep)
    l2, _ = ema(x, ema_decay)
    means = block_means(x, block)
    bhash, babs = simhash(means, proj)
    keys, kabs = simhash(l2, proj)
    idx = retrieve(keys, bhash, np.arange(N), block, top_r)
    l3 = l3_mean(means, idx)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    dh = q.shape[-1] // n_heads
    q_rows = q[:, rows].reshape(B, len(rows), n_heads, dh)
    on = TIER_SETS[tiers]
    k3, v3, a3 = [None] * 3, [None] * 3, [None] * 3
    o = np.zeros((B, len(rows), n_heads, dh))
    for ell, tier in enumerate((x, l2, l3)):
        if not on[ell]:
            continue
        k3[ell], v3[ell] = kv_proj(tier, w_k, w_v, n_kv_heads)
        a3[ell] = attention(q_rows, k3[ell], v3[ell], rows, n_kv_heads)
        o = o + lam[:, rows, ell][:, :, None, None] * a3[ell]
    return dict(q=q, lam=lam, l2=l2, block_means=means, block_hash=bhash, block_abs=babs,
                keys=keys, key_abs=kabs, idx=idx, l3=l3, k3=k3, v3=v3, a3=a3, rows=rows, o=o)


class FullDecodeState(DecodeState):
    """Decode state of full MKA: the three tiers' caches (k3, v3: lists of
    [B,G,t_cap,dh], None for a disabled tier) instead of the fused one."""

    def __init__(self, k3, v3, ema_state, block_acc, means, pos):
        super().__init__(np.zeros(1), np.zeros(1), ema_state, block_acc, means, pos)
        self.k3 = [None if k is None else _f64(k).copy() for k in k3]
        self.v3 = [None if v is None else _f64(v).copy() for v in v3]


def full_decode_init_from_prefill(x, ref, proj, *, block, t_cap):
    """Full-MKA decode state after ``full_prefill`` (``ref``) of x."""
    x = _f64(x)
    B, N, D = x.shape
    nb = N // block

    def grow(c):
        if c is None:
            return None
        out = np.zeros(c.shape[:2] + (t_cap,) + c.shape[3:])
        out[:, :, :N] = c
        return out

    st = FullDecodeState([grow(k) for k in ref["k3"]], [grow(v) for v in ref["v3"]],
                         ref["l2"][:, -1], x[:, nb * block:].sum(axis=1), ref["block_means"], N)
    st.hash, st.hash_abs = simhash(st.means, proj)
    return st


def full_decode_step(st, x_t, w_q, w_k, w_v, w_r1, w_r2, proj, *, n_heads, n_kv_heads,
                     ema_decay, block, top_r, route_mode="soft", tiers="l1l2l3", keep=None):
    """One full-MKA decode step at position t = st.pos: the tiers of the token,
    one K/V row appended to each enabled tier's cache, the three attentions over
    rows 0..t and their lambda-weighted sum.  Block finalisation as in
    ``decode_step``.  Returns q, lam, l2, key, idx, a3 and o ([B, H, dh])."""
    x_t = _f64(x_t)
    B, D = x_t.shape
    t = st.pos
    q = q_proj(x_t, w_q)
    lam = router(q, w_r1, w_r2, route_mode, tiers, keep)
    l2_seq, st.ema_state = ema(x_t[:, None, :], ema_decay, st.ema_state)
    l2 = l2_seq[:, 0]
    st.block_acc = st.block_acc + x_t
    key, kabs = simhash(l2, proj)
    idx = retrieve(key[:, None], st.hash, np.array([t]), block, top_r)
    l3 = l3_mean(st.means, idx)[:, 0]
    dh = q.shape[-1] // n_heads
    qh = q.reshape(B, 1, n_heads, dh)
    on = TIER_SETS[tiers]
    a3 = [None] * 3
    o = np.zeros((B, n_heads, dh))
    for ell, tier in enumerate((x_t, l2, l3)):
        if not on[ell]:
            continue
        k_row, v_row = kv_proj(tier[:, None, :], w_k, w_v, n_kv_heads)
        st.k3[ell][:, :, t] = k_row[:, :, 0]
        st.v3[ell][:, :, t] = v_row[:, :, 0]
        a3[ell] = attention(qh, st.k3[ell], st.v3[ell], np.array([t]), n_kv_heads)[:, 0]
        o = o + lam[:, ell][:, None, None] * a3[ell]
    if (t + 1) % block == 0:
        m = st.block_acc / block
        h, habs = simhash(m, proj)
        st.means = np.concatenate([st.means, m[:, None]], axis=1)
        st.hash = np.concatenate([st.hash, h[:, None]], axis=1)
        st.hash_abs = np.concatenate([st.hash_abs, habs[:, None]], axis=1)
        st.block_acc = np.zeros_like(st.block_acc)
    st.pos = t + 1
    return dict(q=q, lam=lam, l2=l2, key=key, key_abs=kabs, idx=idx[:, 0], l3=l3, a3=a3, o=o)


# --------------------------------------------------------------------------
# Backward of the FastMKA layer (training).  The abstract page's headline is
# training throughput (Tables 1, 2, 6; FlashAttention-2 training in bf16); the
# pages give no backward, so it is the derivative of the forward above taken
# by the chain rule, step by step in reverse.  The SimHash codes and the top-R
# choice are discrete: no gradient flows through them (the retrieved set is a
# constant), nor through a hard router's choice of tiers; the hyperplanes and
# the EMA decay are fixed.  Gradients flow to x and to W_q, W_k, W_v, W_r1,
# W_r2, given dO, the gradient of a loss with respect to the layer output.
# --------------------------------------------------------------------------

def gelu_grad(z):
    """d/dz of z * Phi(z): Phi(z) + z * phi(z)."""
    z = _f64(z)
    return 0.5 * (1.0 + _erf(z / _SQRT2)) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def attention_backward(q, k, v, d_o, n_kv_heads):
    """Gradients of causal GQA attention over every row with respect to q, k, v.

    With S = q k^T / sqrt(dh) (j <= t), P = softmax(S) by rows and O = P v:
    dV = P^T dO, dP = dO v^T, dS = P * (dP - rowsum(dP * P)), dq = dS k / sqrt(dh),
    dk = dS^T q / sqrt(dh); a KV head's gradients sum over its query heads.
    q, d_o: [B, N, H, dh]; k, v: [B, G, N, dh].  Returns dq, dk, dv (same shapes).
    """
    q, k, v, d_o = _f64(q), _f64(k), _f64(v), _f64(d_o)
    B, N, H, dh = q.shape
    scale = 1.0 / math.sqrt(dh)
    future = np.arange(N)[None, :] > np.arange(N)[:, None]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = _group_of(h, H, n_kv_heads)
            s = (q[b, :, h] @ k[b, g].T) * scale
            s[future] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dv[b, g] += p.T @ d_o[b, :, h]
            dp = d_o[b, :, h] @ v[b, g].T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            dq[b, :, h] = (ds @ k[b, g]) * scale
            dk[b, g] += (ds.T @ q[b, :, h]) * scale
    return dq, dk, dv


def ema_adjoint(u, beta):
    """The transpose of the EMA map x -> L2: dx_t = (1 - beta) sum_{s >= t} beta^(s-t) u_s,
    a scan from the last token backwards.  u: [B, N, D]."""
    u = _f64(u)
    out = np.empty_like(u)
    g = np.zeros(u.shape[0:1] + u.shape[2:])
    for t in range(u.shape[1] - 1, -1, -1):
        g = u[:, t] + beta * g
        out[:, t] = (1.0 - beta) * g
    return out


def l3_adjoint(c, idx, n_blocks, n_tokens, block):
    """The transpose of x -> L3 through the block means, with the retrieval fixed:
    each token's c[t] / |S_t| goes to the means of its retrieved blocks, and a
    block mean's gradient spreads evenly (1 / Bs) over the block's tokens.
    c: [B, n, D]; idx: [B, n, R].  Returns the gradient on x [B, n_tokens, D]."""
    c = _f64(c)
    B, n, D = c.shape
    dm = np.zeros((B, n_blocks, D))
    for b in range(B):
        for t in range(n):
            sel = idx[b, t][idx[b, t] >= 0]
            for blk in sel:
                dm[b, blk] += c[b, t] / len(sel)
    dx = np.zeros((B, n_tokens, D))
    for blk in range(n_blocks):
        dx[:, blk * block:(blk + 1) * block] += dm[:, blk][:, None, :] / block
    return dx


def backward(x, w_q, w_k, w_v, w_r1, w_r2, proj, d_o, *, n_heads, n_kv_heads, ema_decay,
             block, top_r, route_mode="soft", tiers="l1l2l3", keep=None):
    """Gradients of sum(O * d_o) for the FastMKA layer over a whole sequence.

    Returns a dict with dx [B,N,D], dw_q, dw_k, dw_v, dw_r1, dw_r2 (the weight
    shapes, [out, in]), and the intermediates dq [B,N,H*dh] (attention plus
    router), dk, dv [B,G,N,dh], dxf [B,N,D], dlam [B,N,3], dz [B,N,3], and the
    forward's dict as ``fwd``.
    """
    x = _f64(x)
    B, N, D = x.shape
    fwd = prefill(x, w_q, w_k, w_v, w_r1, w_r2, proj, n_heads=n_heads, n_kv_heads=n_kv_heads,
                  ema_decay=ema_decay, block=block, top_r=top_r, route_mode=route_mode,
                  tiers=tiers, keep=keep)
    q, lam = fwd["q"], fwd["lam"]
    dh = q.shape[-1] // n_heads
    G = n_kv_heads
    w_q, w_k, w_v, w_r1, w_r2 = (_f64(w) for w in (w_q, w_k, w_v, w_r1, w_r2))
    # attention
    dq_a, dk, dv = attention_backward(q.reshape(B, N, n_heads, dh), fwd["k"], fwd["v"],
                                      _f64(d_o), n_kv_heads)
    dk_t = dk.transpose(0, 2, 1, 3).reshape(B, N, G * dh)  # token-major
    dv_t = dv.transpose(0, 2, 1, 3).reshape(B, N, G * dh)
    # K = X_fused W_k^T, V = X_fused W_v^T
    xf = fwd["x_fused"]
    dxf = dk_t @ w_k + dv_t @ w_v
    dw_k = np.einsum("bnk,bnd->kd", dk_t, xf)
    dw_v = np.einsum("bnk,bnd->kd", dv_t, xf)
    # X_fused = lam1 x + lam2 L2 + lam3 L3
    tiers_v = (x, fwd["l2"], fwd["l3"])
    dlam = np.stack([(dxf * t).sum(axis=-1) for t in tiers_v], axis=-1)
    dx = lam[..., 0:1] * dxf
    dx += ema_adjoint(lam[..., 1:2] * dxf, ema_decay)
    dx += l3_adjoint(lam[..., 2:3] * dxf, fwd["idx"], fwd["block_means"].shape[1], N, block)
    # router: lambda = softmax over the kept tiers of z = GELU(q W_r1^T) W_r2^T
    pre = q @ w_r1.T
    hid = gelu(pre)
    if route_mode == "fixed" or tiers == "l1":
        dz = np.zeros_like(lam)  # lambda does not depend on the router
    else:
        kept = lam > 0.0
        dz = np.where(kept, lam * (dlam - (lam * dlam).sum(axis=-1, keepdims=True)), 0.0)
    dw_r2 = np.einsum("bnc,bnr->cr", dz, hid)
    dpre = (dz @ w_r2) * gelu_grad(pre)
    dw_r1 = np.einsum("bnr,bnq->rq", dpre, q)
    dq = dq_a.reshape(B, N, n_heads * dh) + dpre @ w_r1
    # Q = x W_q^T
    dw_q = np.einsum("bnq,bnd->qd", dq, x)
    dx += dq @ w_q
    return dict(dx=dx, dw_q=dw_q, dw_k=dw_k, dw_v=dw_v, dw_r1=dw_r1, dw_r2=dw_r2, dq=dq, dk=dk,
                dv=dv, dxf=dxf, dlam=dlam, dz=dz, fwd=fwd)

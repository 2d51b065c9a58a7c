"""Pins of the CPU oracle to facts fixed outside itself.

Each test checks one oracle function against a closed form, a special case
that reduces to a textbook or library routine, a brute-force evaluation on a
tiny input, an invariant, or a hand-worked example under tests/golden/.  They
are chosen so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.  CPU only.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mka_oracle as O
from route_kv_memory_amd import inputs as I


def rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- EMA (L2)

def test_ema_closed_form_bruteforce():
    # s_t = (1 - b) * sum_{i <= t} b^(t - i) x_i, evaluated term by term.
    x = rng(1).standard_normal((2, 37, 5))
    beta = 0.9
    l2, final = O.ema(x, beta)
    for bb in range(2):
        for t in range(37):
            ref = [(1 - beta) * sum(beta ** (t - i) * x[bb, i, d] for i in range(t + 1))
                   for d in range(5)]
            np.testing.assert_allclose(l2[bb, t], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(final, l2[:, -1])


def test_ema_constant_input_closed_form():
    # x_t = c for all t  ->  s_t = c (1 - b^(t+1)): pins s_{-1} = 0 and the (1 - b) gain.
    beta, c = 0.99, 2.5
    l2, _ = O.ema(np.full((1, 300, 3), c), beta)
    t = np.arange(300)
    np.testing.assert_allclose(l2[0, :, 1], c * (1 - beta ** (t + 1)), rtol=1e-12)


def test_ema_beta_zero_is_identity():
    x = rng(2).standard_normal((1, 20, 4))
    l2, _ = O.ema(x, 0.0)
    np.testing.assert_array_equal(l2, x)


def test_ema_linear_and_state_carry():
    r = rng(3)
    x = r.standard_normal((1, 50, 6))
    w = r.standard_normal((6, 4))
    a, _ = O.ema(x @ w, 0.95)
    b, _ = O.ema(x, 0.95)
    np.testing.assert_allclose(a, b @ w, rtol=1e-10, atol=1e-12)
    first, st = O.ema(x[:, :17], 0.95)
    rest, _ = O.ema(x[:, 17:], 0.95, state=st)
    np.testing.assert_allclose(np.concatenate([first, rest], 1), b, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------- block means

def test_block_means_ramp_closed_form():
    # x[t, d] = t + 1000 d  ->  mean over block b = b*Bs + (Bs-1)/2 + 1000 d.
    # N is not a multiple of Bs: the trailing partial block has no mean.
    Bs, N, D = 8, 45, 3
    x = (np.arange(N)[:, None] + 1000.0 * np.arange(D)[None, :])[None]
    m = O.block_means(x, Bs)
    assert m.shape == (1, N // Bs, D)
    for b in range(N // Bs):
        np.testing.assert_allclose(m[0, b], b * Bs + (Bs - 1) / 2 + 1000.0 * np.arange(D))


# --------------------------------------------------------------- SimHash

def test_simhash_identity_hyperplanes():
    # With hyperplanes = unit axes, bit j is just [v_j > 0], weight 2^j.
    v = np.array([[0.5, -1.0, 2.0, 0.0, -0.25, 3.0, 1e-9, -7.0]])
    codes, absp = O.simhash(v, np.eye(8))
    expect = sum(1 << j for j in range(8) if v[0, j] > 0)
    assert int(codes[0]) == expect == 0b01100101
    np.testing.assert_array_equal(absp[0], np.abs(v[0]))


def test_simhash_single_hyperplane_bit_position():
    # Only hyperplane 5 is non-zero: the code is 0 or 1 << 5.
    proj = np.zeros((40, 3))
    proj[5] = [1.0, -2.0, 0.5]
    c_pos, _ = O.simhash(np.array([[1.0, 0.0, 0.0]]), proj)
    c_neg, _ = O.simhash(np.array([[0.0, 1.0, 0.0]]), proj)
    assert int(c_pos[0]) == 1 << 5 and int(c_neg[0]) == 0


def test_simhash_invariants():
    r = rng(4)
    proj = r.standard_normal((64, 16))
    v = r.standard_normal((30, 16))
    c, _ = O.simhash(v, proj)
    c2, _ = O.simhash(v * 3.7, proj)  # positive scaling keeps every sign
    np.testing.assert_array_equal(c, c2)
    cn, _ = O.simhash(-v, proj)  # negation flips every non-zero projection
    np.testing.assert_array_equal(cn, ~c)
    c0, _ = O.simhash(np.zeros((1, 16)), proj)  # p = 0 gives bit 0
    assert int(c0[0]) == 0
    # top bit (hyperplane 63) is representable
    assert any(int(code) >> 63 for code in c)


# ------------------------------------------------------------- retrieval

def test_retrieval_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "retrieval_hand.json")))
    n = len(g["positions"])
    keys = np.full((1, n), g["key"], dtype=np.uint64)
    bh = np.array([g["block_codes"]], dtype=np.uint64)
    idx = O.retrieve(keys, bh, np.array(g["positions"]), g["block"], g["top_r"])
    np.testing.assert_array_equal(idx[0], np.array(g["expected"]))


@pytest.mark.parametrize("nbits,block,top_r", [(4, 3, 2), (6, 2, 5), (64, 5, 3)])
def test_retrieval_bruteforce(nbits, block, top_r):
    # Full Python sort of (distance, -b) over the eligible blocks of each token.
    r = rng(nbits)
    N, B = 60, 2
    nb = N // block
    mask = (1 << nbits) - 1
    keys = r.integers(0, 2**63, size=(B, N), dtype=np.uint64) & np.uint64(mask)
    bh = r.integers(0, 2**63, size=(B, nb), dtype=np.uint64) & np.uint64(mask)
    idx = O.retrieve(keys, bh, np.arange(N), block, top_r)
    for b in range(B):
        for t in range(N):
            cand = [(bin(int(keys[b, t]) ^ int(bh[b, j])).count("1"), -j, j)
                    for j in range(t // block)]
            want = [j for _, _, j in sorted(cand)][:top_r]
            want += [-1] * (top_r - len(want))
            assert list(idx[b, t]) == want, (b, t)


def test_retrieval_ties_go_to_most_recent_block():
    # Duplicate block means hash to identical codes; the later block must rank first.
    r = rng(5)
    D, nbits = 12, 32
    proj = r.standard_normal((nbits, D))
    base = r.standard_normal(D)
    means = np.stack([base, r.standard_normal(D), base, base, r.standard_normal(D)])[None]
    bh, _ = O.simhash(means, proj)
    key, _ = O.simhash(base[None, None, :] * 0.3, proj)  # same direction as base
    idx = O.retrieve(key, bh, np.array([5 * 4]), 4, 3)
    assert list(idx[0, 0]) == [3, 2, 0]


# ----------------------------------------------------------------- router

def test_gelu_against_math_erf():
    z = np.linspace(-6, 6, 241)
    ref = [zz * 0.5 * (1 + math.erf(zz / math.sqrt(2))) for zz in z]
    np.testing.assert_allclose(O.gelu(z), ref, rtol=1e-14, atol=1e-15)
    assert O.gelu(np.array([0.0]))[0] == 0.0


def test_router_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "router_hand.json")))
    lam = O.router(np.array(g["q"]), np.array(g["w_r1"]), np.array(g["w_r2"]))
    np.testing.assert_allclose(lam, np.array(g["expected"]), rtol=1e-14)


def test_router_uniform_when_output_layer_zero_and_rows_sum_to_one():
    r = rng(6)
    q = r.standard_normal((5, 16))
    w1 = r.standard_normal((8, 16))
    lam0 = O.router(q, w1, np.zeros((3, 8)))
    np.testing.assert_array_equal(lam0, np.full((5, 3), 1 / 3))
    lam = O.router(q * 20, w1, r.standard_normal((3, 8)))  # large logits: max shift needed
    assert np.all(np.isfinite(lam)) and np.all(lam >= 0) and np.all(lam <= 1)
    np.testing.assert_allclose(lam.sum(-1), 1.0, rtol=1e-14)


def test_q_projection_selects_weight_columns():
    # Weights are stored [out, in]: x = e_i gives q = w_q[:, i].
    w = rng(7).standard_normal((6, 4))
    q = O.q_proj(np.eye(4), w)
    np.testing.assert_array_equal(q, w.T)


# ------------------------------------------------------ L3 mean and fusion

def test_l3_mean_hand_example():
    means = np.array([[[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]]])
    idx = np.array([[[2, 0, -1], [-1, -1, -1], [1, -1, -1]]], dtype=np.int32)
    l3 = O.l3_mean(means, idx)
    np.testing.assert_array_equal(l3[0], [[3.0, 4.0], [0.0, 0.0], [3.0, 4.0]])


def test_fuse_hand_example_and_one_hot():
    l1, l2, l3 = np.array([[4.0]]), np.array([[8.0]]), np.array([[-16.0]])
    lam = np.array([[0.5, 0.25, 0.25]])
    assert O.fuse(lam, l1, l2, l3)[0, 0] == 2.0 + 2.0 - 4.0
    for i, src in enumerate((l1, l2, l3)):
        one = np.zeros((1, 3))
        one[0, i] = 1
        assert O.fuse(one, l1, l2, l3)[0, 0] == src[0, 0]


def test_kv_projection_head_major_split():
    # Head g of the cache holds output columns [g*dh, (g+1)*dh) of X W.
    r = rng(8)
    xf = r.standard_normal((1, 5, 6))
    wk = r.standard_normal((4, 6))  # G=2 heads of dh=2
    wv = r.standard_normal((4, 6))
    k, v = O.kv_proj(xf, wk, wv, 2)
    assert k.shape == (1, 2, 5, 2)
    for g in range(2):
        for t in range(5):
            for j in range(2):
                assert math.isclose(k[0, g, t, j], sum(xf[0, t, d] * wk[g * 2 + j, d] for d in range(6)),
                                    rel_tol=1e-12)
                assert math.isclose(v[0, g, t, j], sum(xf[0, t, d] * wv[g * 2 + j, d] for d in range(6)),
                                    rel_tol=1e-12)


def test_fusion_linearity_second_formula():
    # K = lam1 (X Wk) + lam2 EMA(X Wk) + lam3 mean_S(M Wk): projecting each tier
    # first must give the same K as projecting the fused input.
    s = I.workload("tiny_f32")
    d = I.prefill_inputs(s)
    ref = O.prefill(d["x"], d["w_q"], d["w_k"], d["w_v"], d["w_r1"], d["w_r2"], d["proj"],
                    n_heads=s.n_heads, n_kv_heads=s.n_kv_heads, ema_decay=s.ema_decay,
                    block=s.block, top_r=s.top_r, rows=[0])
    x = d["x"].astype(np.float64)
    wk = d["w_k"].astype(np.float64)
    xk = x @ wk.T
    l2k, _ = O.ema(xk, s.ema_decay)
    mk = ref["block_means"] @ wk.T
    l3k = np.zeros_like(xk)
    for t in range(s.seq):
        sel = [b for b in ref["idx"][0, t] if b >= 0]
        if sel:
            l3k[0, t] = mk[0, sel].mean(0)
    lam = ref["lam"]
    k2 = lam[..., 0:1] * xk + lam[..., 1:2] * l2k + lam[..., 2:3] * l3k
    k2 = k2.reshape(1, s.seq, s.n_kv_heads, s.head_dim).transpose(0, 2, 1, 3)
    np.testing.assert_allclose(ref["k"], k2, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("name,seq", [("tiny_f32", 256), ("small_b2", 96)])
def test_layer_end_to_end_by_an_independent_route(name, seq):
    # The whole layer with a learned (general) lambda and a non-empty L3, built
    # a second way from plain definitions and library routines, none of them
    # the oracle's: lambda by torch's exact GELU and softmax; L2 as the
    # lower-triangular matrix (1 - beta) beta^(t-i); block means by a reshape;
    # codes and ranking by a Python sort of (Hamming distance, -block) over the
    # eligible blocks; K and V by projecting each tier first (linearity of the
    # fusion, reading note, section 3); attention by torch's causal
    # scaled-dot-product attention.  The oracle's output must agree.
    s = I.workload("tiny_f32")
    if name == "small_b2":
        s = s.replace(batch=2, d_model=64, n_heads=4, n_kv_heads=2, block=16, top_r=3,
                      router_hidden=16, hash_bits=24, seed=5)
    s = s.replace(seq=seq)
    d = I.prefill_inputs(s)
    ref = O.prefill(d["x"], d["w_q"], d["w_k"], d["w_v"], d["w_r1"], d["w_r2"], d["proj"],
                    n_heads=s.n_heads, n_kv_heads=s.n_kv_heads, ema_decay=s.ema_decay,
                    block=s.block, top_r=s.top_r)
    x = d["x"].astype(np.float64)
    B, N, D = x.shape
    beta = float(s.ema_decay)
    tx = torch.from_numpy(x)
    q = tx @ torch.from_numpy(d["w_q"].astype(np.float64)).T
    hid = torch.nn.functional.gelu(q @ torch.from_numpy(d["w_r1"].astype(np.float64)).T)
    lam = torch.softmax(hid @ torch.from_numpy(d["w_r2"].astype(np.float64)).T, dim=-1).numpy()
    assert lam.min() > 0.01 and lam.max() < 0.99  # a general router output
    ii = np.arange(N)
    wema = np.where(ii[:, None] >= ii[None, :], (1 - beta) * beta ** (ii[:, None] - ii[None, :]
                                                                       ).astype(np.float64), 0.0)
    l2 = np.einsum("ti,bid->btd", wema, x)
    nb = N // s.block
    means = x[:, :nb * s.block].reshape(B, nb, s.block, D).mean(axis=2)
    p = d["proj"].astype(np.float64)

    def code(v):
        return sum(1 << j for j in range(s.hash_bits) if float(v @ p[j]) > 0.0)

    wk, wv = d["w_k"].astype(np.float64), d["w_v"].astype(np.float64)
    ks, vs = np.zeros((B, N, wk.shape[0])), np.zeros((B, N, wv.shape[0]))
    n_l3 = 0
    for b in range(B):
        bcodes = [code(means[b, j]) for j in range(nb)]
        for t in range(N):
            kc = code(l2[b, t])
            order = sorted(range(t // s.block), key=lambda j: (bin(kc ^ bcodes[j]).count("1"), -j))
            sel = order[:s.top_r]
            l3k = np.mean([means[b, j] @ wk.T for j in sel], axis=0) if sel else 0.0
            l3v = np.mean([means[b, j] @ wv.T for j in sel], axis=0) if sel else 0.0
            n_l3 += bool(sel)
            ks[b, t] = lam[b, t, 0] * (x[b, t] @ wk.T) + lam[b, t, 1] * (l2[b, t] @ wk.T) \
                + lam[b, t, 2] * l3k
            vs[b, t] = lam[b, t, 0] * (x[b, t] @ wv.T) + lam[b, t, 1] * (l2[b, t] @ wv.T) \
                + lam[b, t, 2] * l3v
    assert n_l3 >= B * (N - s.block)  # every token past the first block uses L3
    G, dh, H = s.n_kv_heads, s.head_dim, s.n_heads
    tk = torch.from_numpy(ks).view(B, N, G, dh).transpose(1, 2).repeat_interleave(H // G, 1)
    tv = torch.from_numpy(vs).view(B, N, G, dh).transpose(1, 2).repeat_interleave(H // G, 1)
    tq = q.view(B, N, H, dh).transpose(1, 2)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(ref["o"], o.transpose(1, 2).numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(ref["lam"], lam, rtol=1e-12, atol=0)


# -------------------------------------------------------------- attention

def _bruteforce_attention(q, k, v, n_kv):
    B, N, H, dh = q.shape
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            g = h // (H // n_kv)
            for t in range(N):
                s = [sum(q[b, t, h, d] * k[b, g, j, d] for d in range(dh)) / math.sqrt(dh)
                     for j in range(t + 1)]
                mx = max(s)
                w = [math.exp(si - mx) for si in s]
                z = sum(w)
                for d in range(dh):
                    out[b, t, h, d] = sum(w[j] * v[b, g, j, d] for j in range(t + 1)) / z
    return out


def test_attention_bruteforce_tiny_gqa():
    r = rng(9)
    B, N, H, G, dh = 2, 7, 4, 2, 3
    q = r.standard_normal((B, N, H, dh))
    k = r.standard_normal((B, G, N, dh))
    v = r.standard_normal((B, G, N, dh))
    o = O.attention(q, k, v, np.arange(N), G)
    np.testing.assert_allclose(o, _bruteforce_attention(q, k, v, G), rtol=1e-12, atol=1e-13)


def test_attention_matches_torch_sdpa_on_cpu():
    r = rng(10)
    B, N, H, G, dh = 1, 40, 6, 2, 16
    q = r.standard_normal((B, N, H, dh))
    k = r.standard_normal((B, G, N, dh))
    v = r.standard_normal((B, G, N, dh))
    o = O.attention(q, k, v, np.arange(N), G)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).repeat_interleave(H // G, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(H // G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)


def test_attention_closed_forms():
    r = rng(11)
    B, N, H, G, dh = 1, 9, 4, 2, 8
    q = r.standard_normal((B, N, H, dh))
    v = r.standard_normal((B, G, N, dh))
    k = r.standard_normal((B, G, N, dh))
    o = O.attention(q, k, v, np.arange(N), G)
    # Token 0 attends only to itself.
    for h in range(H):
        np.testing.assert_allclose(o[0, 0, h], v[0, h // 2, 0], rtol=1e-14)
    # Equal keys: flat softmax, output = running mean of the values.
    kc = np.broadcast_to(r.standard_normal(dh), (B, G, N, dh))
    oc = O.attention(q, kc, v, np.arange(N), G)
    for t in range(N):
        np.testing.assert_allclose(oc[0, t, 3], v[0, 1, : t + 1].mean(0), rtol=1e-12, atol=1e-14)
    # Two keys with score a/sqrt(dh) and 0: weight of key 1 is sigmoid(a/sqrt(dh)).
    a = 3.0
    q2 = np.zeros((1, 2, 1, dh)); q2[0, 1, 0, 0] = a
    k2 = np.zeros((1, 1, 2, dh)); k2[0, 0, 1, 0] = 1.0
    v2 = np.zeros((1, 1, 2, dh)); v2[0, 0, 1, 0] = 1.0
    o2 = O.attention(q2, k2, v2, np.arange(2), 1)
    assert math.isclose(o2[0, 1, 0, 0], 1 / (1 + math.exp(-a / math.sqrt(dh))), rel_tol=1e-14)


def test_attention_gqa_groups_are_contiguous():
    # Zero values of KV head 1: exactly query heads 3..5 (of 6, G=2) go to zero.
    r = rng(12)
    B, N, H, G, dh = 1, 5, 6, 2, 4
    q = r.standard_normal((B, N, H, dh))
    k = r.standard_normal((B, G, N, dh))
    v = r.standard_normal((B, G, N, dh))
    v[:, 1] = 0.0
    o = O.attention(q, k, v, np.arange(N), G)
    assert np.all(o[:, :, 3:] == 0.0) and np.all(np.abs(o[:, :, :3]).sum(-1) > 0)


def test_online_max_shift_equals_two_pass():
    r = rng(13)
    B, N, H, G, dh = 1, 150, 4, 2, 8
    q = 4.0 * r.standard_normal((B, N, H, dh))  # peaked softmax: rescaling matters
    k = r.standard_normal((B, G, N, dh))
    v = r.standard_normal((B, G, N, dh))
    rows = np.array([0, 1, 63, 64, 65, 127, 149])
    a = O.attention(q[:, rows], k, v, rows, G)
    b = O.attention_online(q[:, rows], k, v, rows, G, tile=16)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------- whole layer

def _tiny(**kw):
    s = I.workload("tiny_f32")
    d = I.prefill_inputs(s)
    args = dict(n_heads=s.n_heads, n_kv_heads=s.n_kv_heads, ema_decay=s.ema_decay,
                block=s.block, top_r=s.top_r)
    args.update(kw)
    return s, d, args


def test_layer_one_hot_router_is_causal_gqa_attention():
    # lambda = (1, 0, 0): X_fused = X, so the layer is standard causal GQA
    # attention of X W_q against X W_k, X W_v (the pages' "L1 only" case).
    s, d, args = _tiny()
    lam = np.zeros((1, s.seq, 3)); lam[..., 0] = 1.0
    ref = O.prefill(d["x"], d["w_q"], d["w_k"], d["w_v"], d["w_r1"], d["w_r2"], d["proj"],
                    lam_override=lam, **args)
    x = torch.from_numpy(d["x"].astype(np.float64))
    q = (x @ torch.from_numpy(d["w_q"].astype(np.float64)).T).view(1, s.seq, s.n_heads, s.head_dim)
    k = (x @ torch.from_numpy(d["w_k"].astype(np.float64)).T).view(1, s.seq, s.n_kv_heads, s.head_dim)
    v = (x @ torch.from_numpy(d["w_v"].astype(np.float64)).T).view(1, s.seq, s.n_kv_heads, s.head_dim)
    rep = s.n_heads // s.n_kv_heads
    o = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(1, 2), k.transpose(1, 2).repeat_interleave(rep, 1),
        v.transpose(1, 2).repeat_interleave(rep, 1), is_causal=True).transpose(1, 2)
    np.testing.assert_allclose(ref["o"], o.numpy(), rtol=1e-10, atol=1e-12)


def test_layer_is_causal():
    # Changing tokens after t0 leaves every output at positions <= t0 unchanged.
    s, d, args = _tiny()
    t0 = 150
    ref = O.prefill(d["x"], d["w_q"], d["w_k"], d["w_v"], d["w_r1"], d["w_r2"], d["proj"], **args)
    x2 = d["x"].copy()
    x2[:, t0 + 1:] = rng(14).standard_normal(x2[:, t0 + 1:].shape).astype(np.float32)
    alt = O.prefill(x2, d["w_q"], d["w_k"], d["w_v"], d["w_r1"], d["w_r2"], d["proj"], **args)
    for key in ("q", "lam", "l2", "keys", "idx", "l3", "x_fused", "o"):
        np.testing.assert_array_equal(ref[key][:, : t0 + 1], alt[key][:, : t0 + 1], err_msg=key)
    np.testing.assert_array_equal(ref["k"][:, :, : t0 + 1], alt["k"][:, :, : t0 + 1])
    np.testing.assert_array_equal(ref["block_hash"][:, : (t0 + 1) // s.block],
                                  alt["block_hash"][:, : (t0 + 1) // s.block])
    assert not np.array_equal(ref["o"][:, t0 + 1:], alt["o"][:, t0 + 1:])


def test_layer_online_attention_agrees():
    s, d, args = _tiny()
    ref = O.prefill(d["x"], d["w_q"], d["w_k"], d["w_v"], d["w_r1"], d["w_r2"], d["proj"], **args)
    rows = np.array([0, 63, 64, 130, 255])
    q = ref["q"][:, rows].reshape(1, len(rows), s.n_heads, s.head_dim)
    o = O.attention_online(q, ref["k"], ref["v"], rows, s.n_kv_heads)
    np.testing.assert_allclose(o, ref["o"][:, rows], rtol=1e-12, atol=1e-14)


def test_decode_continues_prefill():
    # prefill(128) + 128 decode steps == prefill(256) at positions 128..255,
    # including the two block completions (tokens 191 and 255).
    s, d, args = _tiny()
    w = [d[k] for k in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]
    full = O.prefill(d["x"], *w, **args)
    n1 = 128
    part = O.prefill(d["x"][:, :n1], *w, **args)
    st = O.decode_init_from_prefill(d["x"][:, :n1], part, d["proj"], block=s.block, t_cap=s.seq)
    for t in range(n1, s.seq):
        r = O.decode_step(st, d["x"][:, t], *w, **args)
        np.testing.assert_allclose(r["o"], full["o"][:, t], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(r["lam"], full["lam"][:, t], rtol=1e-12)
        np.testing.assert_allclose(r["l2"], full["l2"][:, t], rtol=1e-12, atol=1e-14)
        np.testing.assert_array_equal(r["idx"], full["idx"][:, t])
        np.testing.assert_array_equal(r["key"], full["keys"][:, t])
    np.testing.assert_allclose(st.k, full["k"], rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(st.means, full["block_means"], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(st.hash, full["block_hash"])


# ------------------------------------------------- routing and tier variants
# Abstract page, Table 10 (fixed lambda = 1/3, hard top-2 / top-1 routing) and
# Table 9 (L1+L2, L1+L3, L1 alone = multi-head attention).

_SUBSETS = {"l1l2l3": [0, 1, 2], "l1l2": [0, 1], "l1l3": [0, 2], "l1": [0]}


@pytest.mark.parametrize("tiers", list(_SUBSETS))
def test_soft_routing_over_a_tier_subset_is_scipy_softmax(tiers):
    from scipy.special import softmax
    z = rng(30).standard_normal((5, 7, 3)) * 3.0
    lam = O.route_weights(z, "soft", tiers)
    on = _SUBSETS[tiers]
    off = [i for i in range(3) if i not in on]
    np.testing.assert_allclose(lam[..., on], softmax(z[..., on], axis=-1), rtol=1e-14, atol=1e-16)
    assert np.all(lam[..., off] == 0.0)


def test_soft_routing_all_tiers_is_the_router_softmax():
    r = rng(31)
    q, w1, w2 = r.standard_normal((4, 16)), r.standard_normal((8, 16)), r.standard_normal((3, 8))
    from scipy.special import softmax
    np.testing.assert_allclose(O.router(q, w1, w2, "soft", "l1l2l3"),
                               softmax(O.router_logits(q, w1, w2), axis=-1), rtol=1e-14)
    np.testing.assert_allclose(O.route_weights(O.router_logits(q, w1, w2)),
                               O.router(q, w1, w2), rtol=1e-14)


@pytest.mark.parametrize("tiers", list(_SUBSETS))
def test_fixed_routing_is_uniform_over_enabled_tiers(tiers):
    z = rng(32).standard_normal((3, 11, 3)) * 10.0
    lam = O.route_weights(z, "fixed", tiers)
    on = _SUBSETS[tiers]
    want = np.zeros(3)
    want[on] = 1.0 / len(on)
    np.testing.assert_array_equal(lam, np.broadcast_to(want, lam.shape))


@pytest.mark.parametrize("mode,k", [("top1", 1), ("top2", 2)])
@pytest.mark.parametrize("tiers", list(_SUBSETS))
def test_hard_routing_bruteforce_over_subsets(mode, k, tiers):
    # Brute force: among the k-subsets of the enabled tiers take the one with
    # the largest logit sum (the top-k set when the logits are distinct), and a
    # scipy softmax over it.
    import itertools
    from scipy.special import softmax
    z = rng(33).standard_normal((60, 3))
    lam = O.route_weights(z, mode, tiers)
    on = _SUBSETS[tiers]
    kk = min(k, len(on))
    for row in range(z.shape[0]):
        best = max(itertools.combinations(on, kk), key=lambda c: sum(z[row, i] for i in c))
        want = np.zeros(3)
        want[list(best)] = softmax(z[row, list(best)])
        np.testing.assert_allclose(lam[row], want, rtol=1e-14, atol=1e-16)


def test_hard_routing_ties_go_to_the_lower_tier():
    z = np.array([[1.0, 1.0, 0.0], [0.0, 2.0, 2.0], [3.0, 3.0, 3.0]])
    np.testing.assert_array_equal(O.route_weights(z, "top1"),
                                  [[1, 0, 0], [0, 1, 0], [1, 0, 0]])
    np.testing.assert_allclose(O.route_weights(z, "top2"),
                               [[0.5, 0.5, 0], [0, 0.5, 0.5], [0.5, 0.5, 0]])
    # L1+L3 with L2 largest: L2 is not a candidate
    np.testing.assert_array_equal(O.route_weights(np.array([[0.0, 9.0, 1.0]]), "top1", "l1l3"),
                                  [[0, 0, 1]])


def test_hard_top1_keeps_the_soft_argmax_and_top2_drops_the_soft_argmin():
    z = rng(34).standard_normal((200, 3))
    soft = O.route_weights(z)
    t1 = O.route_weights(z, "top1")
    np.testing.assert_array_equal(np.argmax(t1, -1), np.argmax(soft, -1))
    assert np.all(t1.max(-1) == 1.0)
    t2 = O.route_weights(z, "top2")
    np.testing.assert_array_equal(t2[np.arange(200), np.argmin(soft, -1)], 0.0)
    # the kept pair keeps the soft ratio
    lo = np.argmin(soft, -1)
    a, b = (lo + 1) % 3, (lo + 2) % 3
    i = np.arange(200)
    np.testing.assert_allclose(t2[i, a] / t2[i, b], soft[i, a] / soft[i, b], rtol=1e-12)


def test_layer_l1_tier_alone_is_causal_gqa_attention_whatever_the_router():
    # Table 9's "L1 only (=MHA)": lambda = (1, 0, 0) for every mode, so the
    # layer is torch's causal attention of X W_q against X W_k, X W_v.
    s, d, args = _tiny()
    x = torch.from_numpy(d["x"].astype(np.float64))
    q = (x @ torch.from_numpy(d["w_q"].astype(np.float64)).T).view(1, s.seq, s.n_heads, s.head_dim)
    k = (x @ torch.from_numpy(d["w_k"].astype(np.float64)).T).view(1, s.seq, s.n_kv_heads, s.head_dim)
    v = (x @ torch.from_numpy(d["w_v"].astype(np.float64)).T).view(1, s.seq, s.n_kv_heads, s.head_dim)
    rep = s.n_heads // s.n_kv_heads
    want = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(1, 2), k.transpose(1, 2).repeat_interleave(rep, 1),
        v.transpose(1, 2).repeat_interleave(rep, 1), is_causal=True).transpose(1, 2).numpy()
    w = [d[n] for n in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]
    for mode in O.ROUTE_MODES:
        ref = O.prefill(d["x"], *w, route_mode=mode, tiers="l1", **args)
        np.testing.assert_allclose(ref["o"], want, rtol=1e-10, atol=1e-12, err_msg=mode)
        np.testing.assert_array_equal(ref["lam"][..., 0], 1.0)


def test_layer_fixed_routing_ignores_the_router_and_equals_a_zero_output_layer():
    # Fixed lambda = 1/3 is the soft router with W_r2 = 0 (equal logits), and
    # it does not depend on W_r1, W_r2 at all.
    s, d, args = _tiny()
    w = [d[n] for n in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]
    fixed = O.prefill(d["x"], *w, route_mode="fixed", **args)
    w0 = list(w)
    w0[4] = np.zeros_like(d["w_r2"])
    zero_out = O.prefill(d["x"], *w0, **args)
    np.testing.assert_allclose(fixed["o"], zero_out["o"], rtol=1e-12, atol=1e-14)
    w1 = list(w)
    w1[3] = rng(35).standard_normal(d["w_r1"].shape)
    other = O.prefill(d["x"], *w1, route_mode="fixed", **args)
    np.testing.assert_array_equal(fixed["o"], other["o"])


def test_layer_hard_top1_fuses_exactly_one_tier_per_token():
    s, d, args = _tiny()
    w = [d[n] for n in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]
    ref = O.prefill(d["x"], *w, route_mode="top1", **args)
    tiers = [np.asarray(d["x"], np.float64), ref["l2"], ref["l3"]]
    pick = np.argmax(ref["lam"], -1)
    for t in range(s.seq):
        np.testing.assert_array_equal(ref["x_fused"][0, t], tiers[pick[0, t]][0, t])


def test_layer_without_l3_ignores_the_hash_index():
    # L1+L2: the output cannot depend on the hyperplanes or on R.
    s, d, args = _tiny()
    w = [d[n] for n in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]
    ref = O.prefill(d["x"], *w, tiers="l1l2", **args)
    w2 = list(w)
    w2[5] = rng(36).standard_normal(d["proj"].shape)
    args2 = dict(args, top_r=1)
    alt = O.prefill(d["x"], *w2, tiers="l1l2", **args2)
    np.testing.assert_array_equal(ref["o"], alt["o"])
    full = O.prefill(d["x"], *w2, **args2)
    assert not np.array_equal(full["o"], ref["o"])


@pytest.mark.parametrize("mode,tiers", [("top2", "l1l3"), ("fixed", "l1l2"), ("soft", "l1")])
def test_decode_continues_prefill_for_variants(mode, tiers):
    s, d, args = _tiny()
    args = dict(args, route_mode=mode, tiers=tiers)
    w = [d[k] for k in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]
    full = O.prefill(d["x"], *w, **args)
    n1 = 180
    part = O.prefill(d["x"][:, :n1], *w, **args)
    st = O.decode_init_from_prefill(d["x"][:, :n1], part, d["proj"], block=s.block, t_cap=s.seq)
    for t in range(n1, s.seq):
        r = O.decode_step(st, d["x"][:, t], *w, **args)
        np.testing.assert_allclose(r["o"], full["o"][:, t], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(r["lam"], full["lam"][:, t], rtol=1e-12, atol=1e-15)


def test_hard_routing_explicit_choice():
    # route_choice is the ranking route_weights uses by default; an explicit
    # kept set gives scipy's softmax over exactly those tiers (the weights of
    # the other side of a tie), and fixed routing ignores it.
    r = rng(38)
    z = r.standard_normal((50, 3))
    for mode in ("top1", "top2"):
        keep = O.route_choice(z, mode)
        np.testing.assert_array_equal(O.route_weights(z, mode, keep=keep), O.route_weights(z, mode))
        assert np.all(keep.sum(-1) == {"top1": 1, "top2": 2}[mode])
    alt = np.zeros((50, 3), dtype=bool)
    alt[:, 1] = alt[:, 2] = True
    lam = O.route_weights(z, "top2", keep=alt)
    want = np.zeros_like(z)
    from scipy.special import softmax

    want[:, 1:] = softmax(z[:, 1:], axis=-1)
    np.testing.assert_allclose(lam, want, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(O.route_weights(z, "fixed", keep=alt), O.route_weights(z, "fixed"))
    # the choice is the float64 ranking of the logits: a gap of 1e-12 decides it
    z2 = np.array([[0.5, 0.5 + 1e-12, 0.1], [0.5 + 1e-12, 0.5, 0.1]])
    np.testing.assert_array_equal(O.route_choice(z2, "top1"),
                                  [[False, True, False], [True, False, False]])


# ----------------------------------------------------- full MKA (three paths)
# Reading note, section 2: O_h = sum_l lambda_l a_l with a_l = softmax(q_h k_l^T) v_l.

def _sdpa(q, k, v, n_heads, n_kv_heads, head_dim):
    """torch's causal attention of q [B,N,H*dh] against head-major k, v [B,G,N,dh]."""
    B, N = q.shape[:2]
    tq = torch.from_numpy(q).view(B, N, n_heads, head_dim).transpose(1, 2)
    rep = n_heads // n_kv_heads
    tk = torch.from_numpy(k).repeat_interleave(rep, 1)
    tv = torch.from_numpy(v).repeat_interleave(rep, 1)
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True) \
        .transpose(1, 2).numpy()


def test_full_mka_paths_are_torch_attention_over_each_tier():
    s, d, args = _tiny()
    w = [d[n] for n in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]
    ref = O.full_prefill(d["x"], *w, **args)
    x = np.asarray(d["x"], np.float64)
    o = np.zeros_like(ref["o"])
    for ell, tier in enumerate((x, ref["l2"], ref["l3"])):
        # the tier's keys and values by explicit head-major products
        kk = (tier @ np.asarray(d["w_k"], np.float64).T).reshape(1, s.seq, s.n_kv_heads, s.head_dim)
        vv = (tier @ np.asarray(d["w_v"], np.float64).T).reshape(1, s.seq, s.n_kv_heads, s.head_dim)
        kk, vv = kk.transpose(0, 2, 1, 3), vv.transpose(0, 2, 1, 3)
        np.testing.assert_allclose(ref["k3"][ell], kk, rtol=1e-12, atol=1e-13)
        a = _sdpa(ref["q"], kk, vv, s.n_heads, s.n_kv_heads, s.head_dim)
        np.testing.assert_allclose(ref["a3"][ell], a, rtol=1e-10, atol=1e-12)
        o += ref["lam"][..., ell][..., None, None] * a
    np.testing.assert_allclose(ref["o"], o, rtol=1e-10, atol=1e-12)
    # three different paths: the mixture is not FastMKA's single attention
    fast = O.prefill(d["x"], *w, **args)
    assert np.abs(fast["o"] - ref["o"]).max() > 1e-4


def test_full_mka_equals_fastmka_when_the_tiers_coincide():
    # beta = 0 makes L2 = x; with L1 and L2 enabled both paths attend over the
    # same K/V, so the mixture and FastMKA's fused attention are both GQA of x.
    s, d, args = _tiny(ema_decay=0.0)
    w = [d[n] for n in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]
    full = O.full_prefill(d["x"], *w, tiers="l1l2", **args)
    fast = O.prefill(d["x"], *w, tiers="l1l2", **args)
    l1 = O.prefill(d["x"], *w, tiers="l1", **args)
    np.testing.assert_allclose(full["o"], fast["o"], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(full["o"], l1["o"], rtol=1e-9, atol=1e-12)
    # and with L1 alone every variant of both is plain GQA
    full1 = O.full_prefill(d["x"], *w, tiers="l1", **args)
    np.testing.assert_allclose(full1["o"], l1["o"], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("mode,tiers", [("soft", "l1l2l3"), ("top1", "l1l3")])
def test_full_mka_decode_continues_prefill(mode, tiers):
    s, d, args = _tiny()
    args = dict(args, route_mode=mode, tiers=tiers)
    w = [d[k] for k in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]
    full = O.full_prefill(d["x"], *w, **args)
    n1 = 180
    part = O.full_prefill(d["x"][:, :n1], *w, **args)
    st = O.full_decode_init_from_prefill(d["x"][:, :n1], part, d["proj"], block=s.block,
                                         t_cap=s.seq)
    for t in range(n1, s.seq):
        r = O.full_decode_step(st, d["x"][:, t], *w, **args)
        np.testing.assert_allclose(r["o"], full["o"][:, t], rtol=1e-10, atol=1e-13)
        np.testing.assert_array_equal(r["idx"], full["idx"][:, t])
    for ell in range(3):
        if full["k3"][ell] is None:
            assert st.k3[ell] is None
        else:
            np.testing.assert_allclose(st.k3[ell], full["k3"][ell], rtol=1e-10, atol=1e-13)
            np.testing.assert_allclose(st.v3[ell], full["v3"][ell], rtol=1e-10, atol=1e-13)


# ------------------------------------------------------------------ backward

def test_gelu_grad_is_torch_autograd():
    z = torch.linspace(-6, 6, 241, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.gelu(z).sum().backward()
    np.testing.assert_allclose(O.gelu_grad(z.detach().numpy()), z.grad.numpy(), rtol=1e-13,
                               atol=1e-15)


def test_attention_backward_is_torch_autograd_of_sdpa():
    r = rng(40)
    B, N, H, G, dh = 2, 37, 4, 2, 8
    q, k, v = r.standard_normal((B, N, H, dh)), r.standard_normal((B, G, N, dh)), \
        r.standard_normal((B, G, N, dh))
    d_o = r.standard_normal((B, N, H, dh))
    dq, dk, dv = O.attention_backward(q, k, v, d_o, G)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(1, 2), tk.repeat_interleave(H // G, 1), tv.repeat_interleave(H // G, 1),
        is_causal=True).transpose(1, 2)
    (o * torch.tensor(d_o)).sum().backward()
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-10, atol=1e-12)


def test_ema_and_l3_adjoints():
    # <A a, b> = <a, A^T b> for the EMA map and for x -> L3 through the block means
    r = rng(41)
    a, c = r.standard_normal((2, 50, 6)), r.standard_normal((2, 50, 6))
    l2, _ = O.ema(a, 0.9)
    assert math.isclose((l2 * c).sum(), (a * O.ema_adjoint(c, 0.9)).sum(), rel_tol=1e-12)
    block, R = 8, 3
    means = O.block_means(a, block)
    codes, _ = O.simhash(means, r.standard_normal((16, 6)))
    keys, _ = O.simhash(l2, r.standard_normal((16, 6)))
    idx = O.retrieve(keys, codes, np.arange(50), block, R)
    l3 = O.l3_mean(means, idx)
    lhs = (l3 * c).sum()
    rhs = (a * O.l3_adjoint(c, idx, means.shape[1], 50, block)).sum()
    assert np.any(idx >= 0) and math.isclose(lhs, rhs, rel_tol=1e-12)


def _fd_layer(mode, tiers):
    s = I.workload("tiny_f32").replace(seq=160)
    d = I.prefill_inputs(s)
    args = dict(n_heads=s.n_heads, n_kv_heads=s.n_kv_heads, ema_decay=s.ema_decay,
                block=s.block, top_r=s.top_r, route_mode=mode, tiers=tiers)
    params = {k: np.asarray(d[k], np.float64) for k in ("x", "w_q", "w_k", "w_v", "w_r1", "w_r2")}
    d_o = rng(42).standard_normal((1, s.seq, s.n_heads, s.head_dim))
    return s, d, args, params, d_o


@pytest.mark.parametrize("mode,tiers", [("soft", "l1l2l3"), ("top2", "l1l3"), ("fixed", "l1l2")])
def test_backward_matches_central_differences(mode, tiers):
    s, d, args, params, d_o = _fd_layer(mode, tiers)
    names = ("x", "w_q", "w_k", "w_v", "w_r1", "w_r2")

    def run(p):
        return O.prefill(p["x"], p["w_q"], p["w_k"], p["w_v"], p["w_r1"], p["w_r2"], d["proj"],
                         **args)

    grads = O.backward(params["x"], params["w_q"], params["w_k"], params["w_v"], params["w_r1"],
                       params["w_r2"], d["proj"], d_o, **args)
    base = run(params)
    r = rng(43)
    eps = 1e-5
    checked = 0
    for name in names:
        g = grads["d" + name if name == "x" else "d" + name.replace("w_", "w_")]
        for _ in range(5):
            i = tuple(int(r.integers(n)) for n in params[name].shape)
            vals = []
            for sign in (1, -1):
                p = {k: v.copy() for k, v in params.items()}
                p[name][i] += sign * eps
                out = run(p)
                # the discrete choices must not move under the perturbation
                assert np.array_equal(out["idx"], base["idx"])
                assert np.array_equal(out["lam"] > 0, base["lam"] > 0)
                vals.append((out["o"] * d_o).sum())
            fd = (vals[0] - vals[1]) / (2 * eps)
            np.testing.assert_allclose(g[i], fd, rtol=2e-6, atol=2e-9, err_msg=f"{name}{i}")
            checked += 1
    assert checked == 30

"""The error bound that certifies SimHash signs computed from bf16 parts.

The GPU computes v . p from bf16 parts of both float32 operands,
x = h + l + r (rows v: h = x with its low 16 bits cleared, l likewise of
x - h; hyperplanes p: h and l rounded to nearest even), as
sum(h_v h_p + h_v l_p + l_v h_p) with float32 accumulation, and trusts the
sign wherever |s| exceeds

    F(n) ||v|| ||p||,
    F(n) = (1 + 2^-6) gamma_n + 2^-14 + 2^-15 + 2^-16 + 2^-21,
    gamma_n = n 2^-23 / (1 - n 2^-23),  n = number of float32 additions.

These checks emulate that arithmetic in NumPy (truncation split, float32
sums in shuffled orders, exact references by math.fsum) on inputs chosen to
make the error large: mantissas just below a power of two (largest
truncation remainders), same-sign terms (no cancellation), and mixed
magnitudes.  They pin the derivation (the constants and the Cauchy-Schwarz
step), not the kernel; the kernel's codes are compared with the oracle's on
the GPU.
"""

import math

import numpy as np
import pytest


def split_trunc(x):
    """Truncated bf16 parts (as float32 values) of a float32 array."""
    x = np.asarray(x, dtype=np.float32)
    h = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    r = (x - h).astype(np.float32)  # exact in float32
    lo = (r.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    return h, lo


def rne_bits(b):
    b = b.astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)


def split_rne(x):
    """bf16 parts rounded to nearest even (as float32 values), as the GPU
    splits the hyperplanes."""
    x = np.asarray(x, dtype=np.float32)
    h = rne_bits(x.view(np.uint32)).view(np.float32)
    r = (x - h).astype(np.float32)  # exact in float32
    lo = rne_bits(r.view(np.uint32)).view(np.float32)
    return h, lo


def factor(n):
    u = 2.0 ** -23
    g = n * u / (1.0 - n * u)
    return (1.0 + 2.0 ** -6) * g + 2.0 ** -14 + 2.0 ** -15 + 2.0 ** -16 + 2.0 ** -21


def fp32_sum(terms, order):
    acc = np.float32(0.0)
    for t in terms[order]:
        acc = np.float32(acc + t)
    return float(acc)


def emulate(v, p, rng, orders=3):
    """Largest |s - v.p| over a few summation orders, and the exact v.p."""
    hv, lv = split_trunc(v)
    hp, lp = split_rne(p)
    # each bf16 x bf16 product is exact in float32
    terms = np.concatenate([(hv * hp).astype(np.float32), (hv * lp).astype(np.float32),
                            (lv * hp).astype(np.float32)])
    exact = math.fsum(float(a) * float(b) for a, b in zip(v.astype(np.float64), p.astype(np.float64)))
    worst = 0.0
    for _ in range(orders):
        worst = max(worst, abs(fp32_sum(terms, rng.permutation(terms.size)) - exact))
    # sorted ascending and descending magnitude: the classical bad orders
    idx = np.argsort(np.abs(terms))
    worst = max(worst, abs(fp32_sum(terms, idx) - exact), abs(fp32_sum(terms, idx[::-1]) - exact))
    return worst, exact, terms.size


def test_split_parts_are_exact_bf16_and_bounded():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(4096), rng.uniform(-1e-30, 1e-30, 64),
                        [1.0, -1.0, 0.0, 3.0e38, 2.0 ** -126]]).astype(np.float32)
    h, lo = split_trunc(x)
    assert np.all((h.view(np.uint32) & 0xFFFF) == 0) and np.all((lo.view(np.uint32) & 0xFFFF) == 0)
    x64, h64, l64 = x.astype(np.float64), h.astype(np.float64), lo.astype(np.float64)
    ax = np.abs(x64)
    assert np.all(np.abs(h64) <= ax)
    assert np.all(np.abs(x64 - h64) <= 2.0 ** -7 * ax)
    assert np.all(np.abs(l64) <= 2.0 ** -7 * ax)
    assert np.all(np.abs(x64 - h64 - l64) <= 2.0 ** -14 * ax)


def test_rne_split_parts_are_exact_bf16_and_bounded():
    rng = np.random.default_rng(7)
    m = np.float32(np.nextafter(np.float32(2.0), np.float32(0.0)))
    x = np.concatenate([rng.standard_normal(4096), np.ldexp(m, rng.integers(-8, 8, 256)),
                        [1.0, -1.0, 0.0, 1.00390625, 1.005859375]]).astype(np.float32)
    h, lo = split_rne(x)
    assert np.all((h.view(np.uint32) & 0xFFFF) == 0) and np.all((lo.view(np.uint32) & 0xFFFF) == 0)
    x64, h64, l64 = x.astype(np.float64), h.astype(np.float64), lo.astype(np.float64)
    ax = np.abs(x64)
    assert np.all(np.abs(x64 - h64) <= 2.0 ** -8 * ax)
    assert np.all(np.abs(l64) <= 2.0 ** -8 * (1 + 2.0 ** -8) * ax)
    assert np.all(np.abs(x64 - h64 - l64) <= 2.0 ** -16 * ax)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert h[-2] == np.float32(1.0)


@pytest.mark.parametrize("kind", ["normal", "below_pow2", "same_sign", "mixed_scale"])
def test_bound_holds(kind):
    rng = np.random.default_rng({"normal": 1, "below_pow2": 2, "same_sign": 3, "mixed_scale": 4}[kind])
    D = 224  # one wave's slice of a 3584-wide row
    for _ in range(6):
        if kind == "normal":
            v = rng.normal(0, 0.07, D)
            p = rng.standard_normal(D)
        elif kind == "below_pow2":
            # mantissa 1.1111111 1111111111111111: the largest truncation remainders
            e = rng.integers(-3, 3, D)
            m = np.float32(np.nextafter(np.float32(2.0), np.float32(0.0)))
            v = np.ldexp(m, e) * rng.choice([-1, 1], D)
            p = np.ldexp(m, rng.integers(-3, 3, D)) * rng.choice([-1, 1], D)
        elif kind == "same_sign":
            m = np.float32(np.nextafter(np.float32(2.0), np.float32(0.0)))
            v = np.full(D, m) * rng.uniform(0.5, 1.0, D)
            p = np.full(D, m) * rng.uniform(0.5, 1.0, D)
        else:
            v = rng.standard_normal(D) * np.exp(rng.uniform(-20, 20, D))
            p = rng.standard_normal(D) * np.exp(rng.uniform(-5, 5, D))
        v = np.asarray(v, dtype=np.float32)
        p = np.asarray(p, dtype=np.float32)
        worst, exact, n = emulate(v, p, rng)
        bound = factor(n) * float(np.linalg.norm(v.astype(np.float64)) *
                                  np.linalg.norm(p.astype(np.float64)))
        assert worst <= bound, (kind, worst, bound)


def test_bound_over_slices_adds_up():
    """Slices summed in float64: the per-slice bounds add, and the sum of
    per-slice norm products is at most the product of the full norms."""
    rng = np.random.default_rng(5)
    D, W = 3584, 16
    v = rng.normal(0, 0.07, D).astype(np.float32)
    p = rng.standard_normal(D).astype(np.float32)
    total, bound = 0.0, 0.0
    for w in range(W):
        sl = slice(w * D // W, (w + 1) * D // W)
        worst, exact, n = emulate(v[sl], p[sl], rng, orders=1)
        total += worst
        bound += factor(n) * float(np.linalg.norm(v[sl].astype(np.float64)) *
                                   np.linalg.norm(p[sl].astype(np.float64)))
    assert total <= bound
    assert bound <= factor(3 * D // W) * float(np.linalg.norm(v.astype(np.float64)) *
                                              np.linalg.norm(p.astype(np.float64))) * (1 + 1e-12)


def test_bound_is_not_vacuous():
    """On the workload's value ranges the certified band is narrow: about one
    projection in a hundred needs the float64 recomputation."""
    rng = np.random.default_rng(6)
    D, W = 3584, 16
    v = rng.normal(0, 0.07, (256, D)).astype(np.float32)
    p = rng.standard_normal((64, D)).astype(np.float32)
    proj = v.astype(np.float64) @ p.astype(np.float64).T
    band = np.zeros_like(proj)
    for w in range(W):
        sl = slice(w * D // W, (w + 1) * D // W)
        band += np.outer(np.linalg.norm(v[:, sl].astype(np.float64), axis=1),
                         np.linalg.norm(p[:, sl].astype(np.float64), axis=1))
    band *= factor(3 * D // W)
    frac = float(np.mean(np.abs(proj) <= band))
    assert 0.0 < frac < 0.03, frac

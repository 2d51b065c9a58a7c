"""Seeded synthetic inputs and workload shapes for the FastMKA layer forward.

This module only draws numbers and casts them to the storage type of a
workload.  It holds none of the layer's arithmetic: block hashes, EMA states,
projections and everything downstream are computed by each side (the HIP
library and the CPU oracle) from the arrays returned here.

Every floating-point array is returned as ``numpy.float32`` holding values that
are exactly representable in the workload's storage type: for bf16 workloads
the fp64 draw is rounded once, to nearest-even at 8 significant bits, so the
float32 array converts to bfloat16 without further rounding; for fp32
workloads the fp64 draw is rounded to float32.  The oracle widens these arrays
to float64; the GPU side converts them to its storage type.

Shapes follow the layer's own layout:

* ``x``     [B, N, D]        token hiddens, token-major
* ``w_q``   [H*dh, D]        query projection, stored [out, in]
* ``w_k``   [G*dh, D]        key projection of the fused input, [out, in]
* ``w_v``   [G*dh, D]        value projection of the fused input, [out, in]
* ``w_r1``  [r, H*dh]        router MLP first layer, [out, in]
* ``w_r2``  [3, r]           router MLP second layer, [out, in]
* ``proj``  [nbits, D]       SimHash hyperplanes, one hyperplane per row (fp32)

Weights are drawn i.i.d. N(0, 1/d_in); hyperplanes i.i.d. N(0, 1); token
hiddens i.i.d. N(0, 1), optionally plus a slow sinusoidal drift along the
sequence (per channel period log-uniform in [2048, 32768] tokens, phase
uniform in [0, 2*pi)).

Per-tensor random streams come from ``numpy.random.SeedSequence(seed).spawn``
in one fixed order (see ``_STREAMS``), so a tensor never changes when another
one is added or resized.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "LayerShape",
    "WORKLOADS",
    "workload",
    "round_bf16",
    "prefill_inputs",
    "decode_inputs",
    "sampled_rows",
    "bf16_bits",
]

# Order of the child streams spawned from a workload's base seed.
_STREAMS = (
    "x",
    "w_q",
    "w_k",
    "w_v",
    "w_r1",
    "w_r2",
    "proj",
    "drift",
    "decode_state",
    "decode_tokens",
    "sampled_rows",
)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Shape and hyper-parameters of one FastMKA layer workload."""

    name: str
    dtype: str  # "f32" or "bf16": storage type of x, weights, q, k, v, o
    batch: int
    seq: int  # tokens per sequence in a prefill call
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    router_hidden: int
    ema_decay: float
    block: int
    hash_bits: int
    top_r: int
    seed: int
    drift: bool = False
    n_sampled: int = 0  # >0: full-size checks look at this many sampled rows
    decode_cached: int = 0  # >0: a decode workload with this many cached tokens
    decode_steps: int = 0
    route_mode: str = "soft"  # "soft", "fixed", "top1", "top2"
    tiers: str = "l1l2l3"  # enabled tiers: "l1l2l3", "l1l2", "l1l3", "l1"

    @property
    def n_blocks(self) -> int:
        return self.seq // self.block

    @property
    def q_width(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def is_decode(self) -> bool:
        return self.decode_cached > 0

    def replace(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


# The workloads.  Shapes of single layers of the models the pages measure
# (Qwen2.5-7B: D=3584, 28 query / 4 KV heads; Llama-3.1-8B: D=4096, 32 / 8),
# plus one tiny fp32 layer that the oracle finishes in well under a second.
WORKLOADS = {
    "tiny_f32": LayerShape(
        name="tiny_f32", dtype="f32", batch=1, seq=256, d_model=128, n_heads=2,
        n_kv_heads=1, head_dim=64, router_hidden=32, ema_decay=0.9, block=64,
        hash_bits=32, top_r=2, seed=0),
    "qwen7b_prefill_4k": LayerShape(
        name="qwen7b_prefill_4k", dtype="bf16", batch=2, seq=4096, d_model=3584,
        n_heads=28, n_kv_heads=4, head_dim=128, router_hidden=64, ema_decay=0.99,
        block=128, hash_bits=64, top_r=4, seed=1),
    "qwen7b_prefill_32k": LayerShape(
        name="qwen7b_prefill_32k", dtype="bf16", batch=1, seq=32768, d_model=3584,
        n_heads=28, n_kv_heads=4, head_dim=128, router_hidden=64, ema_decay=0.99,
        block=128, hash_bits=64, top_r=8, seed=2, drift=True, n_sampled=512),
    "qwen7b_decode_128k": LayerShape(
        name="qwen7b_decode_128k", dtype="bf16", batch=1, seq=1, d_model=3584,
        n_heads=28, n_kv_heads=4, head_dim=128, router_hidden=64, ema_decay=0.99,
        block=128, hash_bits=64, top_r=16, seed=3, decode_cached=131072,
        decode_steps=256),
    "qwen7b_decode_32k_b4": LayerShape(
        name="qwen7b_decode_32k_b4", dtype="bf16", batch=4, seq=1, d_model=3584,
        n_heads=28, n_kv_heads=4, head_dim=128, router_hidden=64, ema_decay=0.99,
        block=128, hash_bits=64, top_r=16, seed=5, decode_cached=32768,
        decode_steps=64),
    "llama8b_prefill_64k": LayerShape(
        name="llama8b_prefill_64k", dtype="bf16", batch=1, seq=65536, d_model=4096,
        n_heads=32, n_kv_heads=8, head_dim=128, router_hidden=64, ema_decay=0.995,
        block=256, hash_bits=64, top_r=16, seed=4, n_sampled=256),
}


def workload(name: str) -> LayerShape:
    return WORKLOADS[name]


def _streams(seed: int) -> dict:
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {k: np.random.default_rng(c) for k, c in zip(_STREAMS, children)}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits, nearest-even).

    Returns float32 holding the rounded values.  Valid for finite values in
    the normal range of bfloat16, which covers every draw made here.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)  # a = m * 2**e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(m * 256.0), e - 8)  # np.rint rounds half to even
    return r.astype(np.float32)


def bf16_bits(a32: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of float32 values that are exact in bfloat16."""
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    bits = a32.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("values are not exactly representable in bfloat16")
    return (bits >> 16).astype(np.uint16)


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def _weights(s: LayerShape, st: dict) -> dict:
    D, qw, kw, r = s.d_model, s.q_width, s.kv_width, s.router_hidden
    out = {}
    for key, shape, d_in in (
        ("w_q", (qw, D), D),
        ("w_k", (kw, D), D),
        ("w_v", (kw, D), D),
        ("w_r1", (r, qw), qw),
        ("w_r2", (3, r), r),
    ):
        out[key] = _cast(st[key].standard_normal(shape) / math.sqrt(d_in), s.dtype)
    out["proj"] = st["proj"].standard_normal((s.hash_bits, D)).astype(np.float32)
    return out


def prefill_inputs(s: LayerShape, seq: int | None = None) -> dict:
    """Seeded inputs of a prefill workload: x, the five weights and proj.

    ``seq`` overrides the sequence length (tokens drawn are the prefix of the
    same stream only when ``seq`` is not larger than the workload's).
    """
    if s.is_decode:
        raise ValueError(f"{s.name} is a decode workload")
    n = s.seq if seq is None else seq
    st = _streams(s.seed)
    z = st["x"].standard_normal((s.batch, n, s.d_model))
    if s.drift:
        period = np.exp(st["drift"].uniform(math.log(2048.0), math.log(32768.0), s.d_model))
        phase = st["drift"].uniform(0.0, 2.0 * math.pi, s.d_model)
        t = np.arange(n, dtype=np.float64)[:, None]
        z += np.sin(2.0 * math.pi * t / period[None, :] + phase[None, :])[None]
    out = {"x": _cast(z, s.dtype)}
    del z
    out.update(_weights(s, st))
    return out


def decode_inputs(s: LayerShape) -> dict:
    """Seeded state and tokens of a decode workload.

    The cached state is synthetic: ``k_cache``/``v_cache`` [B, G, T0, dh] hold
    N(0, 1) values; ``ema_state`` [B, D] is N(0, (1-b)/(1+b)), the stationary
    variance of the EMA of unit noise; ``block_means`` [B, T0/Bs, D] are
    N(0, 1/Bs), the spread of a mean of Bs unit draws; the partial block sum
    is zero because T0 is a multiple of Bs.  ``tokens`` [steps, B, D] are the
    new token hiddens, N(0, 1).  Block hashes are not drawn: each side hashes
    ``block_means`` itself.
    """
    if not s.is_decode:
        raise ValueError(f"{s.name} is not a decode workload")
    if s.decode_cached % s.block:
        raise ValueError("cached length must be a multiple of the block size")
    st = _streams(s.seed)
    B, G, T0, dh, D = s.batch, s.n_kv_heads, s.decode_cached, s.head_dim, s.d_model
    ds = st["decode_state"]
    out = {
        "k_cache": _cast(ds.standard_normal((B, G, T0, dh)), s.dtype),
        "v_cache": _cast(ds.standard_normal((B, G, T0, dh)), s.dtype),
        "ema_state": (ds.standard_normal((B, D))
                      * math.sqrt((1.0 - s.ema_decay) / (1.0 + s.ema_decay))).astype(np.float32),
        "block_means": (ds.standard_normal((B, T0 // s.block, D))
                        / math.sqrt(s.block)).astype(np.float32),
        "block_acc": np.zeros((B, D), np.float32),
        "tokens": _cast(st["decode_tokens"].standard_normal((s.decode_steps, B, D)), s.dtype),
    }
    out.update(_weights(s, st))
    return out


def sampled_rows(s: LayerShape) -> np.ndarray:
    """Sorted query rows checked at full size.

    Always holds 0, Bs-1, Bs, R*Bs, R*Bs+1 and N-1 (the first token, both
    sides of the first block boundary, the first token with R eligible blocks
    and the last token); the rest are drawn uniformly without replacement.
    """
    n = s.seq
    fixed = {0, s.block - 1, s.block, s.top_r * s.block, s.top_r * s.block + 1, n - 1}
    fixed = {r for r in fixed if 0 <= r < n}
    if s.n_sampled <= 0 or s.n_sampled >= n:
        return np.arange(n, dtype=np.int64)
    rng = _streams(s.seed)["sampled_rows"]
    pool = np.setdiff1d(np.arange(n, dtype=np.int64), np.fromiter(fixed, np.int64))
    extra = rng.choice(pool, size=s.n_sampled - len(fixed), replace=False)
    return np.sort(np.concatenate([np.fromiter(fixed, np.int64), extra]))

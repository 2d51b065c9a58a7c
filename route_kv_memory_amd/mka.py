"""Thin ctypes binding of the FastMKA C ABI (``include/mka.h``).

The functions carry the C names and arguments.  Array arguments are torch
tensors on the GPU (contiguous; their device pointer is passed) or ``None``
for a null pointer; ``stream`` defaults to torch's current stream.  Nothing
here computes any part of the layer: it marshals arguments and raises
``MkaError`` on a non-zero status.  The library must be built
(``python -m route_kv_memory_amd.build``); loading fails loudly otherwise.
"""

from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "MkaError", "Dims", "Weights", "State", "Outputs", "lib", "dims", "exported_symbols",
    "header_symbols", "MKA_F32", "MKA_BF16", "MKA_OK", "MKA_ERR_INVALID", "MKA_ERR_UNSUPPORTED",
    "MKA_ERR_WORKSPACE", "MKA_ERR_HIP", "MKA_ROUTE_SOFT", "MKA_ROUTE_FIXED", "MKA_ROUTE_TOP1",
    "MKA_ROUTE_TOP2", "MKA_TIERS_ALL", "MKA_TIERS_L1_L2", "MKA_TIERS_L1_L3", "MKA_TIERS_L1",
    "ROUTE_MODES", "TIER_SETS", "MKA_OP_EMA_SCAN", "MKA_OP_FUSE_KV", "MKA_OP_ATTN_DECODE",
    "MKA_OP_PREFILL", "MKA_OP_DECODE_STEP", "MKA_OP_RETRIEVE", "MKA_OP_INDEX", "MKA_OP_ROUTE",
    "mka_route", "mka_ema_scan", "mka_l3_index", "mka_l3_block_kv", "mka_l3_retrieve",
    "mka_fuse_kv_proj",
    "mka_attn_prefill", "mka_attn_decode", "mka_attn_decode_noalloc",
    "mka_attn_decode_noalloc_limit", "mka_prefill", "mka_decode_step", "TierCache",
    "mka_full_prefill", "mka_full_decode_step", "MKA_OP_FULL_PREFILL", "MKA_OP_FULL_DECODE_STEP",
    "Grads", "mka_backward", "MKA_OP_BACKWARD", "mka_attn_backward", "MKA_OP_ATTN_BACKWARD",
    "mka_workspace_bytes", "mka_status_string", "mka_last_error", "mka_version",
    "mka_probe_mfma_bf16", "mka_probe_stream_read", "PROBE_STREAM_WORKGROUPS",
]

PKG = os.path.dirname(os.path.abspath(__file__))
# MKA_LIB names another build of the library (the host-sanitized one for the
# sanitizer tests); by default the in-tree libmka.so.
LIB_PATH = os.environ.get("MKA_LIB") or os.path.join(PKG, "libmka.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "mka.h")
HEADERS = [HEADER, os.path.join(os.path.dirname(PKG), "include", "mka_probe.h")]

MKA_F32, MKA_BF16 = 0, 1
MKA_ROUTE_SOFT, MKA_ROUTE_FIXED, MKA_ROUTE_TOP1, MKA_ROUTE_TOP2 = range(4)
MKA_TIERS_ALL, MKA_TIERS_L1_L2, MKA_TIERS_L1_L3, MKA_TIERS_L1 = range(4)
ROUTE_MODES = {"soft": MKA_ROUTE_SOFT, "fixed": MKA_ROUTE_FIXED, "top1": MKA_ROUTE_TOP1,
               "top2": MKA_ROUTE_TOP2}
TIER_SETS = {"l1l2l3": MKA_TIERS_ALL, "l1l2": MKA_TIERS_L1_L2, "l1l3": MKA_TIERS_L1_L3,
             "l1": MKA_TIERS_L1}
MKA_OK, MKA_ERR_INVALID, MKA_ERR_UNSUPPORTED, MKA_ERR_WORKSPACE, MKA_ERR_HIP = 0, -1, -2, -3, -4
(MKA_OP_EMA_SCAN, MKA_OP_FUSE_KV, MKA_OP_ATTN_DECODE, MKA_OP_PREFILL, MKA_OP_DECODE_STEP,
 MKA_OP_RETRIEVE, MKA_OP_INDEX, MKA_OP_ROUTE, MKA_OP_FULL_PREFILL, MKA_OP_FULL_DECODE_STEP,
 MKA_OP_BACKWARD, MKA_OP_ATTN_BACKWARD) = range(12)


class MkaError(RuntimeError):
    def __init__(self, fn, status):
        detail = mka_status_string(status)
        if status == MKA_ERR_HIP:
            detail += f" ({mka_last_error()})"
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("seq", ctypes.c_int32), ("d_model", ctypes.c_int32),
        ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("router_hidden", ctypes.c_int32), ("block", ctypes.c_int32), ("hash_bits", ctypes.c_int32),
        ("top_r", ctypes.c_int32), ("ema_decay", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("route_mode", ctypes.c_int32), ("tiers", ctypes.c_int32),
    ]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_q", "w_k", "w_v", "w_r1", "w_r2", "proj")]


class State(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("ema_state", "block_acc", "block_means", "block_hash", "block_kv", "k_cache",
                 "v_cache")] + [
        ("nb_cap", ctypes.c_int32), ("t_cap", ctypes.c_int64), ("page_table", ctypes.c_void_p),
        ("page_size", ctypes.c_int32), ("pages_per_seq", ctypes.c_int32)]


class TierCache(ctypes.Structure):
    _fields_ = [("k_cache", ctypes.c_void_p * 3), ("v_cache", ctypes.c_void_p * 3)]


class Outputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("q", "lambda_", "l2", "key", "idx", "o", "lse")]


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dx", "dw_q", "dw_k", "dw_v", "dw_r1", "dw_r2")]


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_PD = ctypes.POINTER(Dims)

_SIGS = {
    "mka_route": (ctypes.c_int, [_PD, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mka_ema_scan": (ctypes.c_int, [_PD, _P, _I64, _P, _P, _P, _P, _I32, _P, _SZ, _P]),
    "mka_l3_index": (ctypes.c_int, [_PD, _P, _I32, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "mka_l3_block_kv": (ctypes.c_int, [_PD, _P, _I32, _I32, _I32, _P, _P, _P, _P]),
    "mka_l3_retrieve": (ctypes.c_int, [_PD, _P, _P, _P, _I32, _I64, _P, _P, _P, _SZ, _P]),
    "mka_fuse_kv_proj": (ctypes.c_int,
                         [_PD, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _I64, _I64, _P, _SZ, _P]),
    "mka_attn_prefill": (ctypes.c_int, [_PD, _P, _P, _P, _I64, _I64, _P, _P]),
    "mka_attn_decode": (ctypes.c_int, [_PD, _P, _P, _P, _I64, _I64, _P, _P, _SZ, _P]),
    "mka_attn_decode_noalloc": (ctypes.c_int, [_PD, _P, _P, _P, _I64, _I64, _P, _P]),
    "mka_attn_decode_noalloc_limit": (ctypes.c_size_t, []),
    "mka_prefill": (ctypes.c_int, [_PD, _P, _I64, ctypes.POINTER(Weights), ctypes.POINTER(State),
                                   ctypes.POINTER(Outputs), _P, _SZ, _P]),
    "mka_decode_step": (ctypes.c_int, [_PD, _P, _I64, ctypes.POINTER(Weights),
                                       ctypes.POINTER(State), ctypes.POINTER(Outputs), _P, _SZ, _P]),
    "mka_workspace_bytes": (ctypes.c_size_t, [_PD, ctypes.c_int, _I64]),
    "mka_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mka_last_error": (ctypes.c_char_p, []),
    "mka_version": (ctypes.c_char_p, []),
    "mka_full_prefill": (ctypes.c_int, [_PD, _P, _I64, ctypes.POINTER(Weights),
                                        ctypes.POINTER(State), ctypes.POINTER(TierCache),
                                        ctypes.POINTER(Outputs), _P, _SZ, _P]),
    "mka_full_decode_step": (ctypes.c_int, [_PD, _P, _I64, ctypes.POINTER(Weights),
                                            ctypes.POINTER(State), ctypes.POINTER(TierCache),
                                            ctypes.POINTER(Outputs), _P, _SZ, _P]),
    "mka_attn_backward": (ctypes.c_int, [_PD, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mka_backward": (ctypes.c_int, [_PD, _P, ctypes.POINTER(Weights), ctypes.POINTER(State),
                                    ctypes.POINTER(Outputs), _P, ctypes.POINTER(Grads), _P, _SZ,
                                    _P]),
    "mka_probe_mfma_bf16": (ctypes.c_int, [_I32, _I32, _P, _P]),
    "mka_probe_stream_read": (ctypes.c_int, [_P, _SZ, _P, _P]),
}


def lib():
    """Load libmka.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m route_kv_memory_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_symbols() -> list[str]:
    """Function names declared in include/*.h."""
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(mka_\w+)\(", text, re.M)))


def exported_symbols() -> list[str]:
    """Names from the header that the loaded library exports."""
    handle = lib()
    return [n for n in header_symbols() if hasattr(handle, n)]


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, rc):
    if rc != MKA_OK:
        raise MkaError(fn, rc)


def dims(shape, seq=None, batch=None) -> Dims:
    """mka_dims of a ``route_kv_memory_amd.inputs.LayerShape``."""
    return Dims(batch=shape.batch if batch is None else batch,
                seq=shape.seq if seq is None else seq, d_model=shape.d_model,
                n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim,
                router_hidden=shape.router_hidden, block=shape.block, hash_bits=shape.hash_bits,
                top_r=shape.top_r, ema_decay=shape.ema_decay,
                dtype=MKA_BF16 if shape.dtype == "bf16" else MKA_F32,
                route_mode=ROUTE_MODES[shape.route_mode], tiers=TIER_SETS[shape.tiers])


# ----------------------------------------------------------------- C entries

def mka_route(d, x, w_q, w_r1, w_r2, q_out, lambda_out, ws=None, ws_bytes=0, stream=None):
    _check("mka_route", lib().mka_route(ctypes.byref(d), _ptr(x), _ptr(w_q), _ptr(w_r1),
                                        _ptr(w_r2), _ptr(q_out), _ptr(lambda_out), _ptr(ws),
                                        ws_bytes, _stream(stream)))


def mka_ema_scan(d, x, pos0, state_io, block_acc_io, l2_out, block_means, nb_cap, ws=None,
                 ws_bytes=0, stream=None):
    _check("mka_ema_scan", lib().mka_ema_scan(
        ctypes.byref(d), _ptr(x), pos0, _ptr(state_io), _ptr(block_acc_io), _ptr(l2_out),
        _ptr(block_means), nb_cap, _ptr(ws), ws_bytes, _stream(stream)))


def mka_l3_index(d, block_means, nb_cap, first_block, n_blocks, proj, block_hash, ws=None,
                 ws_bytes=0, stream=None):
    _check("mka_l3_index", lib().mka_l3_index(
        ctypes.byref(d), _ptr(block_means), nb_cap, first_block, n_blocks, _ptr(proj),
        _ptr(block_hash), _ptr(ws), ws_bytes, _stream(stream)))


def mka_l3_block_kv(d, block_means, nb_cap, first_block, n_blocks, w_k, w_v, block_kv,
                    stream=None):
    _check("mka_l3_block_kv", lib().mka_l3_block_kv(
        ctypes.byref(d), _ptr(block_means), nb_cap, first_block, n_blocks, _ptr(w_k), _ptr(w_v),
        _ptr(block_kv), _stream(stream)))


def mka_l3_retrieve(d, l2, proj, block_hash, nb_cap, pos0, key_out, idx_out, ws=None, ws_bytes=0,
                    stream=None):
    _check("mka_l3_retrieve", lib().mka_l3_retrieve(
        ctypes.byref(d), _ptr(l2), _ptr(proj), _ptr(block_hash), nb_cap, pos0, _ptr(key_out),
        _ptr(idx_out), _ptr(ws), ws_bytes, _stream(stream)))


def mka_fuse_kv_proj(d, x, l2, block_means, nb_cap, idx, lam, w_k, w_v, k_cache, v_cache, pos0,
                     t_cap, ws, ws_bytes, stream=None):
    _check("mka_fuse_kv_proj", lib().mka_fuse_kv_proj(
        ctypes.byref(d), _ptr(x), _ptr(l2), _ptr(block_means), nb_cap, _ptr(idx), _ptr(lam),
        _ptr(w_k), _ptr(w_v), _ptr(k_cache), _ptr(v_cache), pos0, t_cap, _ptr(ws), ws_bytes,
        _stream(stream)))


def mka_attn_prefill(d, q, k_cache, v_cache, t_cap, pos0, o, stream=None):
    _check("mka_attn_prefill", lib().mka_attn_prefill(
        ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache), t_cap, pos0, _ptr(o),
        _stream(stream)))


def mka_attn_decode(d, q, k_cache, v_cache, t_cap, cache_len, o, ws=None, ws_bytes=0,
                    stream=None):
    _check("mka_attn_decode", lib().mka_attn_decode(
        ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache), t_cap, cache_len, _ptr(o),
        _ptr(ws), ws_bytes, _stream(stream)))


def mka_attn_decode_noalloc(d, q, k_cache, v_cache, t_cap, cache_len, o, stream=None):
    _check("mka_attn_decode_noalloc", lib().mka_attn_decode_noalloc(
        ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache), t_cap, cache_len, _ptr(o),
        _stream(stream)))


def mka_attn_decode_noalloc_limit():
    return lib().mka_attn_decode_noalloc_limit()


def mka_prefill(d, x, pos0, weights, state, outputs, ws, ws_bytes, stream=None):
    _check("mka_prefill", lib().mka_prefill(
        ctypes.byref(d), _ptr(x), pos0, ctypes.byref(weights), ctypes.byref(state),
        ctypes.byref(outputs), _ptr(ws), ws_bytes, _stream(stream)))


def mka_decode_step(d, x, pos, weights, state, outputs, ws, ws_bytes, stream=None):
    _check("mka_decode_step", lib().mka_decode_step(
        ctypes.byref(d), _ptr(x), pos, ctypes.byref(weights), ctypes.byref(state),
        ctypes.byref(outputs), _ptr(ws), ws_bytes, _stream(stream)))


def mka_full_prefill(d, x, pos0, weights, state, tiers, outputs, ws, ws_bytes, stream=None):
    _check("mka_full_prefill", lib().mka_full_prefill(
        ctypes.byref(d), _ptr(x), pos0, ctypes.byref(weights), ctypes.byref(state),
        ctypes.byref(tiers), ctypes.byref(outputs), _ptr(ws), ws_bytes, _stream(stream)))


def mka_full_decode_step(d, x, pos, weights, state, tiers, outputs, ws, ws_bytes, stream=None):
    _check("mka_full_decode_step", lib().mka_full_decode_step(
        ctypes.byref(d), _ptr(x), pos, ctypes.byref(weights), ctypes.byref(state),
        ctypes.byref(tiers), ctypes.byref(outputs), _ptr(ws), ws_bytes, _stream(stream)))


def mka_attn_backward(d, q, k_cache, v_cache, t_cap, o, lse, d_o, dq, dkv, ws, ws_bytes,
                      stream=None):
    _check("mka_attn_backward", lib().mka_attn_backward(
        ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache), t_cap, _ptr(o), _ptr(lse),
        _ptr(d_o), _ptr(dq), _ptr(dkv), _ptr(ws), ws_bytes, _stream(stream)))


def mka_backward(d, x, weights, state, fwd, d_o, grads, ws, ws_bytes, stream=None):
    _check("mka_backward", lib().mka_backward(
        ctypes.byref(d), _ptr(x), ctypes.byref(weights), ctypes.byref(state), ctypes.byref(fwd),
        _ptr(d_o), ctypes.byref(grads), _ptr(ws), ws_bytes, _stream(stream)))


def mka_workspace_bytes(d, op, cache_len=0) -> int:
    return int(lib().mka_workspace_bytes(ctypes.byref(d), op, cache_len))


def mka_status_string(status) -> str:
    return lib().mka_status_string(status).decode()


def mka_last_error() -> str:
    return lib().mka_last_error().decode()


def mka_version() -> str:
    return lib().mka_version().decode()


# ------------------------------------------------------------ peak probes

PROBE_STREAM_WORKGROUPS = 2048  # sink floats mka_probe_stream_read writes


def mka_probe_mfma_bf16(workgroups, iters, sink, stream=None):
    _check("mka_probe_mfma_bf16", lib().mka_probe_mfma_bf16(workgroups, iters, _ptr(sink),
                                                            _stream(stream)))


def mka_probe_stream_read(src, nbytes, sink, stream=None):
    _check("mka_probe_stream_read", lib().mka_probe_stream_read(_ptr(src), nbytes, _ptr(sink),
                                                                _stream(stream)))

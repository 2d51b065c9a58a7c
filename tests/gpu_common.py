"""GPU-side helpers for the parity tests: run the HIP path through the C ABI
and bring results back as numpy arrays."""

from __future__ import annotations

import numpy as np
import torch

from route_kv_memory_amd import mka
from route_kv_memory_amd.layer import Layer, to_device

from .parity import log


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def gpu_prefill(s, inp, *, x=None, seq=None, t_cap=None, nb_cap=None, batch=None, pos0=0,
                layer=None):
    """Whole-layer prefill through mka_prefill; returns (layer, outputs)."""
    n = seq if seq is not None else s.seq
    if layer is None:
        layer = Layer(s, inp, t_cap=t_cap or n, nb_cap=nb_cap or max(1, (t_cap or n) // s.block),
                      batch=batch)
    xs = to_device(inp["x"] if x is None else x, s.dtype)
    log(f"  gpu: mka_prefill {s.name} B={layer.batch} seq={xs.shape[1]} pos0={pos0}")
    out = layer.prefill(xs, pos0=pos0)
    torch.cuda.synchronize()
    return layer, out


def state_np(layer):
    st = layer.st
    return dict(k=to_np(layer.logical_cache("k")), v=to_np(layer.logical_cache("v")),
                means=to_np(st["block_means"]), bhash=to_np(st["block_hash"]).view(np.uint64),
                block_kv=to_np(st["block_kv"]),
                ema=to_np(st["ema_state"]), acc=to_np(st["block_acc"]))


def outputs_np(out):
    o = {k: to_np(v) for k, v in out.items()}
    o["key"] = o["key"].view(np.uint64)
    return o


def dims(s, seq=None, batch=None):
    return mka.dims(s, seq=seq, batch=batch)

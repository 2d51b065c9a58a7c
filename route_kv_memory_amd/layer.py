"""Device buffers of one FastMKA layer, driven through the C ABI.

``Layer`` owns the weights, the decode state (EMA state, partial block sum,
block means and codes, fused KV cache) and per-call output buffers as torch
tensors, and calls ``mka_prefill`` / ``mka_decode_step``.  It allocates and
passes pointers; every step of the layer runs in the HIP library.
"""

from __future__ import annotations

import numpy as np
import torch

from . import mka

_TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}


def to_device(a: np.ndarray, dtype: str | None = None, device="cuda") -> torch.Tensor:
    """float32 numpy values -> device tensor of the storage type (exact for
    values representable in it, which is what the input generators return)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(_TORCH[dtype])
    return t.to(device)


class Layer:
    def __init__(self, shape, weights: dict, *, t_cap: int, nb_cap: int, batch: int | None = None,
                 device="cuda", full: bool = False, page_size: int | None = None,
                 spare_pages: int = 0, page_seed: int = 0):
        self.shape = shape
        self.batch = shape.batch if batch is None else batch
        self.device = device
        self.t_cap, self.nb_cap = int(t_cap), int(nb_cap)
        dt = shape.dtype
        self.tdtype = _TORCH[dt]
        self.w = {k: to_device(weights[k], dt, device) for k in ("w_q", "w_k", "w_v", "w_r1", "w_r2")}
        self.w["proj"] = to_device(weights["proj"], None, device)
        self.weights = mka.Weights(**{k: v.data_ptr() for k, v in self.w.items()})
        B, D, G, dh = self.batch, shape.d_model, shape.n_kv_heads, shape.head_dim
        z = dict(device=device)
        # Paged cache: t_cap rounds up to whole pages; the pool holds every
        # sequence's pages (plus spares) in a seeded random order.
        self.page_size = page_size
        if page_size:
            pps = -(-self.t_cap // page_size)
            self.t_cap = pps * page_size
            n_pages = B * pps + spare_pages
            perm = np.random.default_rng(page_seed).permutation(n_pages)[: B * pps]
            self.page_table = torch.from_numpy(perm.astype(np.int32).reshape(B, pps)).to(device)
            cache_shape = (n_pages, G, page_size, dh)
        else:
            self.page_table = None
            cache_shape = (B, G, self.t_cap, dh)
        self.st = {
            "ema_state": torch.zeros(B, D, dtype=torch.float32, **z),
            "block_acc": torch.zeros(B, D, dtype=torch.float32, **z),
            "block_means": torch.zeros(B, self.nb_cap, D, dtype=torch.float32, **z),
            "block_hash": torch.zeros(B, self.nb_cap, dtype=torch.int64, **z),
            "block_kv": torch.zeros(B, self.nb_cap, 2 * G * dh, dtype=torch.float32, **z),
            "k_cache": torch.zeros(cache_shape, dtype=self.tdtype, **z),
            "v_cache": torch.zeros(cache_shape, dtype=self.tdtype, **z),
        }
        self.state = mka.State(nb_cap=self.nb_cap, t_cap=self.t_cap,
                               **{k: v.data_ptr() for k, v in self.st.items()})
        if page_size:
            self.state.page_table = self.page_table.data_ptr()
            self.state.page_size = page_size
            self.state.pages_per_seq = self.page_table.shape[1]
        self._ws = None
        # full MKA: one K/V cache per memory tier (tier 0 = L1, 1 = L2, 2 = L3)
        self.kv3 = None
        if full:
            self.kv3 = {c: [torch.zeros(B, G, self.t_cap, dh, dtype=self.tdtype, **z)
                            for _ in range(3)] for c in ("k", "v")}
            tc = mka.TierCache()
            for i in range(3):
                tc.k_cache[i] = self.kv3["k"][i].data_ptr()
                tc.v_cache[i] = self.kv3["v"][i].data_ptr()
            self.tier_cache = tc

    def index_blocks(self, first: int, n: int, stream=None) -> None:
        """Codes and projections of block means first .. first+n-1 (already in
        ``st["block_means"]``): what a prefill leaves for the blocks it completes."""
        d = self.dims(1)
        ws = self.workspace(mka.mka_workspace_bytes(d, mka.MKA_OP_INDEX, n))
        st = self.st
        mka.mka_l3_index(d, st["block_means"], self.nb_cap, first, n, self.w["proj"],
                         st["block_hash"], ws, ws.numel(), stream)
        mka.mka_l3_block_kv(d, st["block_means"], self.nb_cap, first, n, self.w["w_k"],
                            self.w["w_v"], st["block_kv"], stream)

    def dims(self, seq: int) -> mka.Dims:
        return mka.dims(self.shape, seq=seq, batch=self.batch)

    def outputs(self, seq: int) -> dict:
        s, B, z = self.shape, self.batch, dict(device=self.device)
        return {
            "q": torch.empty(B, seq, s.n_heads, s.head_dim, dtype=self.tdtype, **z),
            "lambda": torch.empty(B, seq, 3, dtype=torch.float32, **z),
            "l2": torch.empty(B, seq, s.d_model, dtype=torch.float32, **z),
            "key": torch.empty(B, seq, dtype=torch.int64, **z),
            "idx": torch.empty(B, seq, s.top_r, dtype=torch.int32, **z),
            "o": torch.empty(B, seq, s.n_heads, s.head_dim, dtype=self.tdtype, **z),
            "lse": torch.empty(B, seq, s.n_heads, dtype=torch.float32, **z),
        }

    @staticmethod
    def _out_struct(out: dict) -> mka.Outputs:
        return mka.Outputs(q=out["q"].data_ptr(), lambda_=out["lambda"].data_ptr(),
                           l2=out["l2"].data_ptr(), key=out["key"].data_ptr(),
                           idx=out["idx"].data_ptr(), o=out["o"].data_ptr(),
                           lse=out["lse"].data_ptr() if "lse" in out else None)

    def workspace(self, nbytes: int) -> torch.Tensor:
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def prefill(self, x: torch.Tensor, pos0: int = 0, out: dict | None = None, stream=None) -> dict:
        seq = x.shape[1]
        d = self.dims(seq)
        out = self.outputs(seq) if out is None else out
        need = mka.mka_workspace_bytes(d, mka.MKA_OP_PREFILL)
        ws = self.workspace(need)
        mka.mka_prefill(d, x, pos0, self.weights, self.state, self._out_struct(out), ws,
                        ws.numel(), stream)
        return out

    def decode_step(self, x_t: torch.Tensor, pos: int, out: dict | None = None, stream=None) -> dict:
        d = self.dims(1)
        out = self.outputs(1) if out is None else out
        need = mka.mka_workspace_bytes(d, mka.MKA_OP_DECODE_STEP, pos + 1)
        ws = self.workspace(need)
        mka.mka_decode_step(d, x_t, pos, self.weights, self.state, self._out_struct(out), ws,
                            ws.numel(), stream)
        return out

    def full_prefill(self, x: torch.Tensor, pos0: int = 0, out: dict | None = None,
                     stream=None) -> dict:
        """Full MKA (three attention paths) over x; the layer needs ``full=True``."""
        seq = x.shape[1]
        d = self.dims(seq)
        out = self.outputs(seq) if out is None else out
        ws = self.workspace(mka.mka_workspace_bytes(d, mka.MKA_OP_FULL_PREFILL))
        mka.mka_full_prefill(d, x, pos0, self.weights, self.state, self.tier_cache,
                             self._out_struct(out), ws, ws.numel(), stream)
        return out

    def full_decode_step(self, x_t: torch.Tensor, pos: int, out: dict | None = None,
                         stream=None) -> dict:
        d = self.dims(1)
        out = self.outputs(1) if out is None else out
        ws = self.workspace(mka.mka_workspace_bytes(d, mka.MKA_OP_FULL_DECODE_STEP, pos + 1))
        mka.mka_full_decode_step(d, x_t, pos, self.weights, self.state, self.tier_cache,
                                 self._out_struct(out), ws, ws.numel(), stream)
        return out

    def logical_cache(self, which: str) -> torch.Tensor:
        """The K or V cache as [B, G, t_cap, dh], gathered through the page
        table when the cache is paged."""
        c = self.st[f"{which}_cache"]
        if self.page_table is None:
            return c
        B, pps = self.page_table.shape
        pages = c[self.page_table.long().reshape(-1)]  # [B*pps, G, P, dh]
        G, P, dh = pages.shape[1:]
        return pages.reshape(B, pps, G, P, dh).permute(0, 2, 1, 3, 4).reshape(B, G, pps * P, dh)

    def load_cache(self, which: str, rows: torch.Tensor) -> None:
        """Write rows [B, G, n, dh] as cache rows 0 .. n-1 (through the page
        table when the cache is paged)."""
        c = self.st[f"{which}_cache"]
        n = rows.shape[2]
        if self.page_table is None:
            c[:, :, :n].copy_(rows)
            return
        P = self.page_size
        pt = self.page_table.long()
        for p in range(-(-n // P)):
            r0, r1 = p * P, min(n, (p + 1) * P)
            c[pt[:, p], :, : r1 - r0] = rows[:, :, r0:r1].to(c.dtype)

    def grads(self, seq: int) -> dict:
        """float32 gradient buffers of x and the weights."""
        s, B, z = self.shape, self.batch, dict(device=self.device, dtype=torch.float32)
        return {
            "dx": torch.empty(B, seq, s.d_model, **z),
            "dw_q": torch.empty(s.q_width, s.d_model, **z),
            "dw_k": torch.empty(s.kv_width, s.d_model, **z),
            "dw_v": torch.empty(s.kv_width, s.d_model, **z),
            "dw_r1": torch.empty(s.router_hidden, s.q_width, **z),
            "dw_r2": torch.empty(3, s.router_hidden, **z),
        }

    def backward(self, x: torch.Tensor, out: dict, d_o: torch.Tensor, grads: dict | None = None,
                 stream=None) -> dict:
        """Gradients of sum(O * d_o) after ``prefill(x, 0, out)`` (the saved forward)."""
        seq = x.shape[1]
        d = self.dims(seq)
        grads = self.grads(seq) if grads is None else grads
        ws = self.workspace(mka.mka_workspace_bytes(d, mka.MKA_OP_BACKWARD))
        g = mka.Grads(**{k: v.data_ptr() for k, v in grads.items()})
        mka.mka_backward(d, x, self.weights, self.state, self._out_struct(out), d_o, g, ws,
                         ws.numel(), stream)
        return grads

"""Host-side logic of route_kv_memory_amd.layer (CPU tensors, no GPU): the paged
cache's page table and the round trip of rows through it."""

import numpy as np
import torch

from route_kv_memory_amd import inputs as I
from route_kv_memory_amd import mka
from route_kv_memory_amd.layer import Layer


def test_paged_layer_tables_and_round_trip():
    s = I.workload("tiny_f32").replace(batch=3)
    inp = I.prefill_inputs(s)
    lay = Layer(s, inp, t_cap=300, nb_cap=4, device="cpu", page_size=64, spare_pages=4,
                page_seed=2)
    assert lay.t_cap == 320 and lay.page_table.shape == (3, 5)
    pt = lay.page_table.numpy()
    assert len(set(pt.ravel())) == pt.size and pt.min() >= 0 and pt.max() < 3 * 5 + 4
    assert lay.st["k_cache"].shape == (19, s.n_kv_heads, 64, s.head_dim)
    assert (lay.state.page_size, lay.state.pages_per_seq, lay.state.t_cap) == (64, 5, 320)
    rows = torch.randn(3, s.n_kv_heads, 250, s.head_dim)
    lay.load_cache("v", rows)
    assert torch.equal(lay.logical_cache("v")[:, :, :250], rows)
    # row t of sequence b sits at row t % 64 of pool page pt[b][t // 64]
    b, t = 2, 201
    assert torch.equal(lay.st["v_cache"][pt[b, t // 64], :, t % 64], rows[b, :, t])


def test_contiguous_layer_has_no_page_table():
    s = I.workload("tiny_f32")
    lay = Layer(s, I.prefill_inputs(s), t_cap=256, nb_cap=4, device="cpu")
    assert lay.page_table is None and lay.state.page_table is None
    assert lay.st["k_cache"].shape == (1, s.n_kv_heads, 256, s.head_dim)
    assert ctypes_size_ok()


def ctypes_size_ok():
    # mka_state: 7 pointers, nb_cap (padded), t_cap, page_table, page_size, pages_per_seq
    import ctypes
    return ctypes.sizeof(mka.State) == 7 * 8 + 8 + 8 + 8 + 4 + 4

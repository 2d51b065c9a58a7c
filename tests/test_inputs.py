"""Seeded input generators: determinism, storage-type rounding, shapes."""

import numpy as np
import torch

from route_kv_memory_amd import inputs as I


def test_round_bf16_matches_bit_rounding_and_torch():
    r = np.random.default_rng(0)
    x32 = (r.standard_normal(100000) * np.exp(r.uniform(-20, 20, 100000))).astype(np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    rne = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint32) << 16
    ref = rne.astype(np.uint32).view(np.float32)
    got = I.round_bf16(x32.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(got, torch.from_numpy(x32).to(torch.bfloat16).float().numpy())
    assert np.all(I.bf16_bits(got) == (got.view(np.uint32) >> 16))


def test_generators_are_deterministic_and_shaped():
    s = I.workload("tiny_f32")
    a, b = I.prefill_inputs(s), I.prefill_inputs(s)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    assert a["x"].shape == (1, 256, 128) and a["w_q"].shape == (128, 128)
    assert a["w_r1"].shape == (32, 128) and a["w_r2"].shape == (3, 32)
    assert a["proj"].shape == (32, 128) and a["proj"].dtype == np.float32
    q = I.workload("qwen7b_prefill_4k").replace(seq=64)
    x = I.prefill_inputs(q)["x"]
    assert np.all(I.round_bf16(x.astype(np.float64)) == x)  # already bf16-exact
    # weights are N(0, 1/d_in)
    assert abs(np.std(I.prefill_inputs(q)["w_q"]) * np.sqrt(3584) - 1) < 0.01


def test_sampled_rows_hold_the_fixed_rows():
    s = I.workload("llama8b_prefill_64k")
    rows = I.sampled_rows(s)
    assert len(rows) == 256 and np.all(np.diff(rows) > 0)
    for r in (0, 255, 256, 16 * 256, 16 * 256 + 1, 65535):
        assert r in rows


def test_drift_gives_block_structure():
    s = I.workload("qwen7b_prefill_32k").replace(seq=2048)
    x = I.prefill_inputs(s)["x"].astype(np.float64)[0]
    m = x.reshape(16, 128, -1).mean(1)
    c = np.corrcoef(m)
    assert np.mean(c[np.arange(15), np.arange(1, 16)]) > 0.5  # neighbouring blocks agree


def test_decode_state_shapes():
    s = I.workload("qwen7b_decode_128k").replace(decode_cached=1024, decode_steps=3)
    d = I.decode_inputs(s)
    assert d["k_cache"].shape == (1, 4, 1024, 128)
    assert d["block_means"].shape == (1, 8, 3584)
    assert d["tokens"].shape == (3, 1, 3584)
    assert np.all(d["block_acc"] == 0)

"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function that include/mka.h declares, and rejects bad arguments with
the documented status codes before launching anything."""

import ctypes

import pytest
import torch

from route_kv_memory_amd import inputs as I
from route_kv_memory_amd import mka


def test_library_exports_every_declared_symbol():
    declared = mka.header_symbols()
    assert len(declared) >= 13
    assert mka.exported_symbols() == declared
    assert "gfx950" in mka.mka_version()


def test_status_strings():
    assert mka.mka_status_string(mka.MKA_OK) == "ok"
    for code in (mka.MKA_ERR_INVALID, mka.MKA_ERR_UNSUPPORTED, mka.MKA_ERR_WORKSPACE,
                 mka.MKA_ERR_HIP):
        assert mka.mka_status_string(code) not in ("ok", "unknown status")
    assert mka.mka_status_string(12345) == "unknown status"


FAKE = 1 << 40  # aligned, non-null, never dereferenced: every call below is rejected first


def _d(**kw):
    d = mka.dims(I.workload("qwen7b_prefill_4k"))
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, mka.MKA_ERR_INVALID),
    ("seq", 0, mka.MKA_ERR_INVALID),
    ("n_kv_heads", 3, mka.MKA_ERR_INVALID),       # 28 % 3 != 0
    ("hash_bits", 65, mka.MKA_ERR_INVALID),
    ("hash_bits", 0, mka.MKA_ERR_INVALID),
    ("ema_decay", 1.0, mka.MKA_ERR_INVALID),
    ("ema_decay", -0.1, mka.MKA_ERR_INVALID),
    ("dtype", 7, mka.MKA_ERR_INVALID),
    ("route_mode", 4, mka.MKA_ERR_INVALID),
    ("route_mode", -1, mka.MKA_ERR_INVALID),
    ("tiers", 4, mka.MKA_ERR_INVALID),
    ("tiers", -1, mka.MKA_ERR_INVALID),
    ("head_dim", 96, mka.MKA_ERR_UNSUPPORTED),
    ("top_r", 33, mka.MKA_ERR_UNSUPPORTED),
    ("d_model", 3584 + 32, mka.MKA_ERR_UNSUPPORTED),  # bf16 needs D % 64 == 0
])
def test_bad_dims_rejected(field, value, code):
    d = _d(**{field: value})
    with pytest.raises(mka.MkaError) as e:
        mka.mka_route(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, stream=0)
    assert e.value.status == code


def test_null_and_misaligned_pointers_rejected():
    d = _d()
    with pytest.raises(mka.MkaError) as e:
        mka.mka_route(d, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, stream=0)
    assert e.value.status == mka.MKA_ERR_INVALID
    with pytest.raises(mka.MkaError) as e:
        mka.mka_attn_prefill(d, FAKE + 2, FAKE, FAKE, 4096, 0, FAKE, stream=0)
    assert e.value.status == mka.MKA_ERR_INVALID


def test_range_checks_rejected():
    d = _d()
    # cache too short for pos0 + seq
    with pytest.raises(mka.MkaError) as e:
        mka.mka_attn_prefill(d, FAKE, FAKE, FAKE, 4095, 0, FAKE, stream=0)
    assert e.value.status == mka.MKA_ERR_INVALID
    # decode needs seq == 1 and 1 <= cache_len <= t_cap
    with pytest.raises(mka.MkaError) as e:
        mka.mka_attn_decode(d, FAKE, FAKE, FAKE, 10, 5, FAKE, FAKE, 1 << 20, stream=0)
    assert e.value.status == mka.MKA_ERR_INVALID
    d1 = _d(seq=1)
    with pytest.raises(mka.MkaError) as e:
        mka.mka_attn_decode(d1, FAKE, FAKE, FAKE, 10, 11, FAKE, FAKE, 1 << 20, stream=0)
    assert e.value.status == mka.MKA_ERR_INVALID
    # too few block means for the blocks completed in this call
    with pytest.raises(mka.MkaError) as e:
        mka.mka_ema_scan(d, FAKE, 0, FAKE, FAKE, FAKE, FAKE, 31, FAKE, 1 << 30, stream=0)
    assert e.value.status == mka.MKA_ERR_INVALID
    # the index range must fit in nb_cap
    with pytest.raises(mka.MkaError) as e:
        mka.mka_l3_index(d, FAKE, 32, 30, 3, FAKE, FAKE, FAKE, 1 << 30, stream=0)
    assert e.value.status == mka.MKA_ERR_INVALID
    with pytest.raises(mka.MkaError) as e:
        mka.mka_l3_block_kv(d, FAKE, 32, 30, 3, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == mka.MKA_ERR_INVALID
    with pytest.raises(mka.MkaError) as e:  # null projected-means buffer
        mka.mka_l3_block_kv(d, FAKE, 32, 0, 3, FAKE, FAKE, None, stream=0)
    assert e.value.status == mka.MKA_ERR_INVALID


def test_workspace_sizes_and_rejection():
    d = _d()
    ema = mka.mka_workspace_bytes(d, mka.MKA_OP_EMA_SCAN)
    fuse = mka.mka_workspace_bytes(d, mka.MKA_OP_FUSE_KV)
    # X_fused in bf16, then the two transposed bf16 planes of up to 256 block
    # means per sequence that the matrix-core L3 path stages
    assert fuse == 2 * 4096 * 3584 * 2 + 2 * 2 * 3584 * 256 * 2
    assert ema == 2 * 4 * 2 * (4096 // 64) * 3584       # chunk carries, 2 floats
    retr = mka.mka_workspace_bytes(d, mka.MKA_OP_RETRIEVE)
    idx = mka.mka_workspace_bytes(d, mka.MKA_OP_INDEX, 33)
    # prefill: the EMA scan and block index (auxiliary stream) run beside the
    # main stream's route, retrieval and fusion, so their regions add up; the
    # key codes' hyperplane split (bf16 hi/lo parts and 16 slice norms per
    # hyperplane, prepared on the auxiliary stream) has a region of its own
    prep = 2 * 64 * 3584 * 2 + 16 * 64 * 8
    assert mka.mka_workspace_bytes(d, mka.MKA_OP_PREFILL) == max(ema, idx) + max(retr, fuse) + prep
    assert idx > 0  # few blocks: the projections are split over d_model
    dd = mka.dims(I.workload("qwen7b_decode_128k"))
    dec = mka.mka_workspace_bytes(dd, mka.MKA_OP_ATTN_DECODE, 131073)
    chunks = 256 // 4  # the split's 131072 rows: one chunk per CU over the 4 KV heads
    assert dec >= 4 * 28 * chunks * (128 + 2)
    assert mka.mka_workspace_bytes(dd, mka.MKA_OP_DECODE_STEP, 131073) >= dec
    with pytest.raises(mka.MkaError) as e:
        mka.mka_ema_scan(d, FAKE, 0, FAKE, FAKE, FAKE, FAKE, 32, FAKE, ema - 1, stream=0)
    assert e.value.status == mka.MKA_ERR_WORKSPACE
    with pytest.raises(mka.MkaError) as e:
        mka.mka_fuse_kv_proj(d, FAKE, FAKE, FAKE, 32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                             4096, FAKE, fuse - 1, stream=0)
    assert e.value.status == mka.MKA_ERR_WORKSPACE
    assert mka.mka_workspace_bytes(_d(batch=0), mka.MKA_OP_PREFILL) == 0


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="launch failure is only safe without a GPU")
def test_launch_without_device_reports_hip_error():
    # A fully valid call on a host with no GPU must fail with MKA_ERR_HIP, not crash.
    d = mka.dims(I.workload("tiny_f32"))
    with pytest.raises(mka.MkaError) as e:
        mka.mka_attn_prefill(d, FAKE, FAKE, FAKE, 256, 0, FAKE, stream=0)
    assert e.value.status == mka.MKA_ERR_HIP
    assert mka.mka_last_error() != ""


def test_routing_fields_follow_the_header():
    # mka_dims ends with route_mode and tiers; zero means the full method.
    assert [f[0] for f in mka.Dims._fields_][-2:] == ["route_mode", "tiers"]
    assert ctypes.sizeof(mka.Dims) == 14 * 4
    d = mka.dims(I.workload("tiny_f32"))
    assert (d.route_mode, d.tiers) == (mka.MKA_ROUTE_SOFT, mka.MKA_TIERS_ALL)
    text = open(mka.HEADER).read()
    for name in ("MKA_ROUTE_SOFT = 0", "MKA_ROUTE_FIXED = 1", "MKA_ROUTE_TOP1 = 2",
                 "MKA_ROUTE_TOP2 = 3", "MKA_TIERS_ALL = 0", "MKA_TIERS_L1_L2 = 1",
                 "MKA_TIERS_L1_L3 = 2", "MKA_TIERS_L1 = 3"):
        assert name in text
        key, val = name.split(" = ")
        assert getattr(mka, key) == int(val)


def test_probe_arguments_rejected():
    lib = mka.lib()
    assert lib.mka_probe_mfma_bf16(0, 10, FAKE, None) == mka.MKA_ERR_INVALID
    assert lib.mka_probe_mfma_bf16(4, 0, FAKE, None) == mka.MKA_ERR_INVALID
    assert lib.mka_probe_mfma_bf16(4, 10, None, None) == mka.MKA_ERR_INVALID
    assert lib.mka_probe_stream_read(FAKE + 8, 1024, FAKE, None) == mka.MKA_ERR_INVALID
    assert lib.mka_probe_stream_read(FAKE, 1000, FAKE, None) == mka.MKA_ERR_INVALID
    assert lib.mka_probe_stream_read(None, 1024, FAKE, None) == mka.MKA_ERR_INVALID


def test_full_mka_arguments_rejected():
    d = _d()
    w = mka.Weights(*([FAKE] * 6))
    st = mka.State(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, nb_cap=64, t_cap=8192)
    out = mka.Outputs(*([FAKE] * 6))
    tc = mka.TierCache()  # null caches
    with pytest.raises(mka.MkaError) as e:
        mka.mka_full_prefill(d, FAKE, 0, w, st, tc, out, FAKE, 1 << 40, 0)
    assert e.value.status == mka.MKA_ERR_INVALID
    for i in range(3):
        tc.k_cache[i] = FAKE
        tc.v_cache[i] = FAKE
    with pytest.raises(mka.MkaError) as e:  # workspace too small
        mka.mka_full_prefill(d, FAKE, 0, w, st, tc, out, FAKE, 16, 0)
    assert e.value.status == mka.MKA_ERR_WORKSPACE
    with pytest.raises(mka.MkaError) as e:  # decode needs seq == 1
        mka.mka_full_decode_step(d, FAKE, 10, w, st, tc, out, FAKE, 1 << 40, 0)
    assert e.value.status == mka.MKA_ERR_INVALID
    # L1 alone needs only the first tier's cache
    d1 = _d(seq=1, tiers=mka.MKA_TIERS_L1)
    tc2 = mka.TierCache()
    tc2.k_cache[0] = FAKE
    with pytest.raises(mka.MkaError) as e:  # v_cache[0] missing
        mka.mka_full_decode_step(d1, FAKE, 10, w, st, tc2, out, FAKE, 1 << 40, 0)
    assert e.value.status == mka.MKA_ERR_INVALID
    assert mka.mka_workspace_bytes(d, mka.MKA_OP_FULL_PREFILL) > 0
    assert mka.mka_workspace_bytes(d1, mka.MKA_OP_FULL_DECODE_STEP, 100) > 0
    assert mka.mka_workspace_bytes(d, mka.MKA_OP_FULL_DECODE_STEP, 100) == 0  # seq != 1


def test_paged_state_rejections():
    d = _d(seq=128)
    w = mka.Weights(*([FAKE] * 6))
    out = mka.Outputs(*([FAKE] * 6))

    def state(**kw):
        st = mka.State(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, nb_cap=64, t_cap=8192)
        st.page_table, st.page_size, st.pages_per_seq = FAKE, 256, 32
        for k, v in kw.items():
            setattr(st, k, v)
        return st

    for bad in (dict(page_size=100), dict(page_size=32), dict(pages_per_seq=0),
                dict(pages_per_seq=31), dict(page_table=FAKE + 2)):
        with pytest.raises(mka.MkaError) as e:
            mka.mka_prefill(d, FAKE, 0, w, state(**bad), out, FAKE, 1 << 40, 0)
        assert e.value.status == mka.MKA_ERR_INVALID, bad
    tc = mka.TierCache()
    for i in range(3):
        tc.k_cache[i] = FAKE
        tc.v_cache[i] = FAKE
    with pytest.raises(mka.MkaError) as e:  # the full-MKA tier caches are contiguous
        mka.mka_full_prefill(d, FAKE, 0, w, state(), tc, out, FAKE, 1 << 40, 0)
    assert e.value.status == mka.MKA_ERR_UNSUPPORTED


def test_noalloc_decode_rejects_requests_beyond_its_scratch():
    # 4 MiB of device scratch: one 128K Qwen-shaped sequence needs 0.93 MB of
    # split partials; 128 sequences of 64 single-head groups need 4.26 MB.
    assert mka.mka_attn_decode_noalloc_limit() == 4 << 20
    d = mka.dims(I.workload("qwen7b_decode_128k"), seq=1)
    assert mka.mka_workspace_bytes(d, mka.MKA_OP_ATTN_DECODE, 131073) <= 4 << 20
    big = mka.dims(I.workload("qwen7b_decode_128k").replace(batch=128, n_heads=64, n_kv_heads=64,
                                                             d_model=8192), seq=1)
    need = mka.mka_workspace_bytes(big, mka.MKA_OP_ATTN_DECODE, 4096)
    assert need > 4 << 20
    with pytest.raises(mka.MkaError) as e:
        mka.mka_attn_decode_noalloc(big, FAKE, FAKE, FAKE, 4096, 4096, FAKE, stream=0)
    assert e.value.status == mka.MKA_ERR_WORKSPACE
    assert "scratch" in mka.mka_last_error()
    with pytest.raises(mka.MkaError) as e:  # the usual argument checks come first
        mka.mka_attn_decode_noalloc(d, FAKE, FAKE, FAKE, 10, 11, FAKE, stream=0)
    assert e.value.status == mka.MKA_ERR_INVALID

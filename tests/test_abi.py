"""The C-ABI library: it loads, exports every entry point its header
declares, and rejects bad host-visible arguments before any HIP call (so
these checks run without a GPU).  No test here launches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


@pytest.fixture(scope="module")
def rp():
    import replayssm_persistent_rssm_amd as rp
    return rp


POOL_HEADER = os.path.join(ROOT, "include", "rssm_pool.h")


def declared_functions(headers):
    names = set()
    for h in headers:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(rssm_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_entry_point(rp):
    """librssm_materialize exports every entry point its headers declare."""
    names = declared_functions([h for h in HEADERS if h != POOL_HEADER])
    assert names == sorted(rp.EXPORTS)
    for n in names:
        assert hasattr(rp.lib(), n), n


def test_pool_helper_is_a_separate_library(rp):
    """rssm_pool.h's allocating helpers live in librssm_pool alone: the
    operation's library exports none of them."""
    names = declared_functions([POOL_HEADER])
    assert names == sorted(rp.POOL_EXPORTS)
    for n in names:
        assert hasattr(rp.pool_lib(), n), n
        assert not hasattr(rp.lib(), n), f"{n} is exported by the operation's library"


def _desc(rp, **kw):
    base = dict(num_layers=48, batch=256, num_heads=256, heads_per_group=32, dim=64, dstate=128, max_window=8,
                ring_buffer_len=16, state_dtype="bf16", input_dtype="bf16")
    base.update(kw)
    return rp.make_desc(**base)


def _fake_tables(rp, **override):
    # Aligned, non-NULL addresses that are never dereferenced: every call below
    # fails host validation before touching the device.
    t = rp.RssmTables(**{f: 0x10000 for f, _ in rp.RssmTables._fields_})
    for k, v in override.items():
        setattr(t, k, v)
    return t


BAD_DESCS = [
    (dict(num_layers=0), 1, "num_layers"),
    (dict(batch=0), 1, "batch"),
    (dict(num_heads=0), 1, "num_heads"),
    (dict(heads_per_group=3), 1, "divide"),
    (dict(max_window=0), 1, "max_window"),
    (dict(max_window=17), 1, "max_window"),
    (dict(ring_buffer_len=0), 1, "ring_buffer_len"),
    (dict(philox_rounds=-1), 1, "philox_rounds"),
    (dict(max_workgroups=-1), 1, "max_workgroups"),
    (dict(state_dtype=9), 1, "state_dtype"),
    (dict(input_dtype="i8"), 2, "input_dtype"),
    (dict(matrixA_dtype="bf16"), 2, "a_dtype"),
    (dict(state_dtype="i8", dim=32), 1, "one-byte"),
    (dict(dim=32, dstate=64), 2, "no compiled instance"),
    (dict(num_layers=2**20, batch=2**20, num_heads=2**10), 1, "2^40"),
]


@pytest.mark.parametrize("kw,status,text", BAD_DESCS)
def test_bad_scalars_rejected(rp, kw, status, text):
    d = _desc(rp, **kw)
    t = _fake_tables(rp)
    st = rp.lib().rssm_materialize(ctypes.byref(d), ctypes.byref(t), None)
    assert st == status
    assert text in rp.rssm_last_error()


def test_null_and_misaligned_tables_rejected(rp):
    d = _desc(rp)
    assert rp.lib().rssm_materialize(ctypes.byref(d), None, None) == 1
    assert rp.lib().rssm_materialize(None, None, None) == 1
    for field in ("state_ptrs", "dt_slot_strides", "A_ptrs", "src_slots", "active_request_indices"):
        t = _fake_tables(rp, **{field: None})
        assert rp.lib().rssm_materialize(ctypes.byref(d), ctypes.byref(t), None) == 1
        assert field in rp.rssm_last_error()
    t = _fake_tables(rp, state_ptrs=0x10004)
    assert rp.lib().rssm_materialize(ctypes.byref(d), ctypes.byref(t), None) == 1
    assert "aligned" in rp.rssm_last_error()
    t = _fake_tables(rp, ring_start=0x10002)
    assert rp.lib().rssm_materialize(ctypes.byref(d), ctypes.byref(t), None) == 1


def test_quantized_state_needs_scales_and_sr_needs_seed(rp):
    d = _desc(rp, state_dtype="f8e4m3")
    t = _fake_tables(rp, scale_ptrs=None)
    assert rp.lib().rssm_materialize(ctypes.byref(d), ctypes.byref(t), None) == 1
    assert "scale" in rp.rssm_last_error()
    d = _desc(rp, state_dtype="bf16", philox_rounds=10)
    t = _fake_tables(rp, rand_seed=None)
    assert rp.lib().rssm_materialize(ctypes.byref(d), ctypes.byref(t), None) == 1
    assert "rand_seed" in rp.rssm_last_error()


def test_python_binding_rejects_out_of_range_scalars(rp):
    with pytest.raises(ValueError):
        _desc(rp, num_heads=2**31)        # never narrowed
    with pytest.raises(ValueError):
        rp.dtype_code("int4")


def test_debug_encode_rows_validation(rp):
    d = _desc(rp, state_dtype="i8", dstate=16, dim=16)
    st = rp.lib().rssm_debug_encode_rows(ctypes.byref(d), 0x10000, 0x10000, None, 0x10000, 0x10000, 4, None)
    assert st == 2
    d = _desc(rp, state_dtype="bf16")
    assert rp.lib().rssm_debug_encode_rows(ctypes.byref(d), None, None, None, None, None, -1, None) == 1
    assert rp.lib().rssm_debug_encode_rows(ctypes.byref(d), None, None, None, None, None, 0, None) == 0


def test_debug_row_scales_validation(rp):
    lib = rp.lib()
    assert lib.rssm_debug_row_scales(rp.RSSM_BF16, 0x10000, 0x10000, 0x10000, 4, None) == 1
    assert "one-byte" in rp.rssm_last_error()
    assert lib.rssm_debug_row_scales(rp.RSSM_I8, 0x10000, 0x10000, 0x10000, -1, None) == 1
    assert lib.rssm_debug_row_scales(rp.RSSM_F8E4M3, None, 0x10000, 0x10000, 4, None) == 1
    assert lib.rssm_debug_row_scales(rp.RSSM_I8, None, None, None, 0, None) == 0


def test_caller_examples_from_the_pages(rp):
    rows = [l.split() for l in open(os.path.join(ROOT, "tests", "golden", "caller_examples.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 2
    for pos, buffered, period, expected in rows:
        assert rp.checkpoint_prefix_len(int(pos), int(buffered), int(period)) == int(expected)
    assert rp.checkpoint_prefix_len(120, 3, 128) is None


def test_algorithmic_bytes_formula():
    """Per written (layer, request): 2*H*dim*dstate*s_b state bytes plus
    k*(H*dim + G*dstate)*i_b + k*H*4 ring bytes (for the large bf16
    workload: 8,388,608 + k*35,840), plus H*4 bytes of A per layer."""
    import rssm_inputs as ri
    import rssm_harness as hx
    spec = ri.CONFIGS["large_bf16"]
    meta = ri.make_meta(spec, np.random.default_rng(0), n_active=3)
    k = meta.prefix[meta.active[:3]]
    want = sum(spec.L * (8_388_608 + int(kk) * 35_840) for kk in k) + spec.L * spec.H * 4
    assert hx.algorithmic_bytes(spec, meta) == want


def test_checkpoints_entry_point_validation(rp):
    d = _desc(rp)
    t = _fake_tables(rp)
    for n in (0, -1, 5):
        assert rp.lib().rssm_materialize_checkpoints(ctypes.byref(d), ctypes.byref(t), n, None) == 1
        assert "num_checkpoints" in rp.rssm_last_error()
    # the multi-checkpoint instances cover the 64x128 tile only
    d16 = _desc(rp, dim=16, dstate=16)
    assert rp.lib().rssm_materialize_checkpoints(ctypes.byref(d16), ctypes.byref(t), 2, None) == 2
    assert "multi-checkpoint" in rp.rssm_last_error()
    assert rp.lib().rssm_materialize_checkpoints(ctypes.byref(d), None, 2, None) == 1
    assert rp.lib().rssm_materialize_checkpoints(None, ctypes.byref(t), 2, None) == 1
    d8 = _desc(rp, state_dtype="i8")
    t8 = _fake_tables(rp, scale_slot_strides=None)
    assert rp.lib().rssm_materialize_checkpoints(ctypes.byref(d8), ctypes.byref(t8), 3, None) == 1
    assert "scale" in rp.rssm_last_error()


def test_checkpoint_byte_count(rp):
    import rssm_harness as hx
    import rssm_inputs as ri
    spec = ri.CONFIGS["large_bf16"]
    meta = ri.make_meta(spec, np.random.default_rng(1002))
    dst, pre = hx.flush_and_checkpoint_tables(meta)
    # every (layer, request) reads its state once, writes it twice and
    # replays the longer prefix
    tile = spec.H * spec.dim * spec.dstate * 2
    ring = spec.H * spec.dim * 2 + spec.G * spec.dstate * 2 + spec.H * 4
    want = sum(spec.L * (3 * tile + int(meta.prefix[b]) * ring) for b in range(spec.B)) + spec.L * spec.H * 4
    assert hx.checkpoint_bytes(spec, meta, dst, pre) == want


def _gdn_desc(rp, **kw):
    base = dict(num_layers=48, slots=512, num_v_heads=32, num_k_heads=16, window=8, batch=256, use_l2norm=1,
                null_block_id=-1, max_workgroups=0)
    base.update(kw)
    return rp.RssmGdnDesc(**base)


def _gdn_tables(rp, **override):
    t = rp.RssmGdnTables(**{f: 0x10000 for f, _ in rp.RssmGdnTables._fields_})
    for k, v in override.items():
        setattr(t, k, v)
    return t


BAD_GDN = [
    (dict(num_layers=0), "num_layers"), (dict(slots=0), "slots"), (dict(num_k_heads=3), "divide"),
    (dict(num_v_heads=0), "divide"), (dict(window=0), "window"), (dict(window=17), "window"),
    (dict(batch=-1), "batch"), (dict(use_l2norm=2), "use_l2norm"), (dict(null_block_id=-2), "null_block_id"),
    (dict(max_workgroups=-1), "max_workgroups"), (dict(num_layers=2**20, slots=2**20, num_v_heads=2, num_k_heads=1), "2^40"),
]


@pytest.mark.parametrize("kw,text", BAD_GDN)
def test_gdn_bad_scalars_rejected(rp, kw, text):
    d = _gdn_desc(rp, **kw)
    t = _gdn_tables(rp)
    assert rp.lib().rssm_gdn_commit(ctypes.byref(d), ctypes.byref(t), None) == 1
    assert text in rp.rssm_last_error()


def test_gdn_tables_rejected(rp):
    d = _gdn_desc(rp)
    assert rp.lib().rssm_gdn_commit(ctypes.byref(d), None, None) == 1
    assert rp.lib().rssm_gdn_commit(None, None, None) == 1
    for field in ("checkpoint_state", "rawk_cache", "beta_cache", "accept_lens"):
        t = _gdn_tables(rp, **{field: None})
        assert rp.lib().rssm_gdn_commit(ctypes.byref(d), ctypes.byref(t), None) == 1
        assert field in rp.rssm_last_error()
    t = _gdn_tables(rp, rawv_cache=0x10008)
    assert rp.lib().rssm_gdn_commit(ctypes.byref(d), ctypes.byref(t), None) == 1
    assert "aligned" in rp.rssm_last_error()
    t = _gdn_tables(rp, track_steps=None)
    assert rp.lib().rssm_gdn_commit(ctypes.byref(d), ctypes.byref(t), None) == 1
    assert "track" in rp.rssm_last_error()
    # an empty batch enqueues nothing and touches no device
    assert rp.lib().rssm_gdn_commit(ctypes.byref(_gdn_desc(rp, batch=0)), ctypes.byref(_gdn_tables(rp)), None) == 0


def _ssu_desc(rp, **kw):
    H, R = 256, 16
    base = dict(batch=256, num_heads=H, heads_per_group=32, dim=64, dstate=128, ring_buffer_len=R, tokens=4,
                num_slots=512, pad_slot_id=-1, state_dtype=1, input_dtype=1, dt_softplus=1, max_workgroups=0,
                state_slot_stride=H * 64 * 128, x_slot_stride=R * H * 64, B_slot_stride=R * 8 * 128,
                dt_slot_stride=R * H)
    base.update(kw)
    return rp.RssmSsuDesc(**base)


def _ssu_tables(rp, **override):
    t = rp.RssmSsuTables(**{f: 0x10000 for f, _ in rp.RssmSsuTables._fields_})
    for k, v in override.items():
        setattr(t, k, v)
    return t


BAD_SSU = [
    (dict(batch=-1), 1, "batch"), (dict(num_heads=0), 1, "num_heads"), (dict(heads_per_group=3), 1, "divide"),
    (dict(tokens=0), 1, "tokens"), (dict(tokens=9), 1, "tokens"), (dict(ring_buffer_len=3), 1, "ring_buffer_len"),
    (dict(num_slots=0), 1, "num_slots"), (dict(dt_softplus=2), 1, "dt_softplus"),
    (dict(max_workgroups=-1), 1, "max_workgroups"), (dict(state_dtype=7), 1, "dtype"),
    (dict(state_dtype=3), 2, "f32, bf16 or f16"), (dict(input_dtype=4), 2, "f32, bf16 or f16"),
    (dict(dim=16, dstate=16), 2, "dim=16"), (dict(state_slot_stride=100), 1, "stride"),
    (dict(x_slot_stride=16 * 256 * 64 - 1), 1, "stride"), (dict(state_slot_stride=256 * 64 * 128 + 3), 1, "16 bytes"),
    (dict(ring_buffer_len=2**20, x_slot_stride=2**20 * 256 * 64, dt_slot_stride=2**20 * 256,
          B_slot_stride=2**20 * 8 * 128), 1, "2^31"),
]


@pytest.mark.parametrize("kw,status,text", BAD_SSU)
def test_ssu_bad_scalars_rejected(rp, kw, status, text):
    d = _ssu_desc(rp, **kw)
    assert rp.lib().rssm_ssu_decode(ctypes.byref(d), ctypes.byref(_ssu_tables(rp)), None) == status
    assert text in rp.rssm_last_error()


def test_ssu_tables_rejected(rp):
    d = _ssu_desc(rp)
    assert rp.lib().rssm_ssu_decode(ctypes.byref(d), None, None) == 1
    assert rp.lib().rssm_ssu_decode(None, None, None) == 1
    for field in ("state", "x_ring", "B_ring", "dt_ring", "A", "x_new", "B_new", "C_new", "dt_new", "y", "slots",
                  "ring_start", "num_buffered"):
        t = _ssu_tables(rp, **{field: None})
        assert rp.lib().rssm_ssu_decode(ctypes.byref(d), ctypes.byref(t), None) == 1
        assert field in rp.rssm_last_error()
    for field in ("state", "B_ring", "C_new"):
        t = _ssu_tables(rp, **{field: 0x10008})
        assert rp.lib().rssm_ssu_decode(ctypes.byref(d), ctypes.byref(t), None) == 1
        assert "aligned" in rp.rssm_last_error()
    t = _ssu_tables(rp, z=0x10001)
    assert rp.lib().rssm_ssu_decode(ctypes.byref(d), ctypes.byref(t), None) == 1
    # the optional vectors may be absent; an empty batch enqueues nothing and touches no device
    t = _ssu_tables(rp, D=None, dt_bias=None, z=None, x_new=None, y=None)
    assert rp.lib().rssm_ssu_decode(ctypes.byref(_ssu_desc(rp, batch=0)), ctypes.byref(t), None) == 0


def test_ssu_byte_count():
    """The decode step's algorithmic bytes, written out for one live request
    with n = 3 and one padded request."""
    import rssm_harness as hx
    import rssm_inputs as ri
    spec = ri.with_(ri.SSU_CONFIGS["ssu_small"], B=2, T=2, has_z=True)
    H, G, T, dim, ds = spec.H, spec.G, spec.T, spec.dim, spec.dstate
    want = 3 * H * 4 + H * dim * ds * 2 + 3 * (H * (dim * 2 + 4) + G * ds * 2)
    want += T * (H * (2 * dim * 2 + 4) + 2 * G * ds * 2) + T * H * dim * 4 + T * (H * (dim * 2 + 4) + G * ds * 2)
    assert hx.ssu_bytes(spec, [7, spec.pad_slot_id], [3, 5]) == want


def test_pool_alloc_validation(rp):
    """Host validation of the pool allocator, before any HIP call."""
    out = ctypes.c_void_p(123)
    assert rp.pool_lib().rssm_pool_alloc(ctypes.c_uint64(1 << 20), None, None) == 1
    assert rp.pool_lib().rssm_pool_alloc(ctypes.c_uint64(0), ctypes.byref(out), None) == 1
    assert out.value is None
    assert rp.pool_lib().rssm_pool_free(None) == 0

"""ctypes binding of librssm_materialize (argument marshalling only).

Every entry point has the C name from ``include/rssm_materialize.h``.  Torch
supplies device memory and streams; the binding checks host-visible tensor
metadata (device, dtype, shape, contiguity), converts tensors to device
addresses and calls the library.  There is no CPU fallback: if the library is
missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librssm_materialize.so")
# the contiguous-pool placement helper (rssm_pool.h): a library of its own,
# outside the operation's boundary
POOL_LIB_PATH = os.path.join(_PKG, "librssm_pool.so")

RSSM_F32, RSSM_BF16, RSSM_F16, RSSM_I8, RSSM_F8E4M3 = 0, 1, 2, 3, 4
RSSM_OK, RSSM_ERR_INVALID_ARGUMENT, RSSM_ERR_UNSUPPORTED, RSSM_ERR_HIP = 0, 1, 2, 3
EXPORTS = ("rssm_materialize", "rssm_materialize_checkpoints", "rssm_last_error", "rssm_materialize_launch_config",
           "rssm_debug_encode_rows", "rssm_debug_row_scales", "rssm_gdn_commit", "rssm_ssu_decode")
POOL_EXPORTS = ("rssm_pool_alloc", "rssm_pool_free", "rssm_torch_pool_alloc", "rssm_torch_pool_free")
RSSM_MAX_CHECKPOINTS = 4
RSSM_SSU_MAX_TOKENS = 8
RSSM_SSU_MAX_REPLAY = 16
_INT32_MAX = 2**31 - 1


class RssmError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"rssm status {status}: {message}")
        self.status = status


class RssmDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_layers", "batch", "num_heads", "heads_per_group", "dim", "dstate", "max_window",
        "ring_buffer_len", "pad_slot_id", "philox_rounds", "state_dtype", "input_dtype", "a_dtype",
        "max_workgroups")]


_I64P = ctypes.c_void_p
_I32P = ctypes.c_void_p


class RssmTables(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "state_ptrs", "state_slot_strides", "x_ptrs", "x_slot_strides", "B_ptrs", "B_slot_strides",
        "dt_ptrs", "dt_slot_strides", "A_ptrs", "scale_ptrs", "scale_slot_strides", "src_slots", "dst_slots",
        "ring_start", "replay_prefix_len", "active_request_indices", "rand_seed")]


class RssmGdnDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_layers", "slots", "num_v_heads", "num_k_heads", "window", "batch", "use_l2norm", "null_block_id",
        "max_workgroups")]


class RssmGdnTables(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "checkpoint_state", "rawv_cache", "rawk_cache", "g_cache", "beta_cache", "state_indices", "accept_lens",
        "track_state_indices", "track_steps")]


class RssmSsuDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_heads", "heads_per_group", "dim", "dstate", "ring_buffer_len", "tokens", "num_slots",
        "pad_slot_id", "state_dtype", "input_dtype", "dt_softplus", "max_workgroups")] + [
        (n, ctypes.c_int64) for n in ("state_slot_stride", "x_slot_stride", "B_slot_stride", "dt_slot_stride")]


class RssmSsuTables(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "state", "x_ring", "B_ring", "dt_ring", "A", "D", "dt_bias", "x_new", "B_new", "C_new", "dt_new", "z", "y",
        "slots", "ring_start", "num_buffered")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built. Build it with `python -m replayssm_persistent_rssm_amd.build` "
            "(or __graft_entry__.build()); there is no fallback path.")
    lib = ctypes.CDLL(LIB_PATH)
    lib.rssm_materialize.argtypes = [ctypes.POINTER(RssmDesc), ctypes.POINTER(RssmTables), ctypes.c_void_p]
    lib.rssm_materialize.restype = ctypes.c_int
    lib.rssm_materialize_checkpoints.argtypes = [ctypes.POINTER(RssmDesc), ctypes.POINTER(RssmTables),
                                                 ctypes.c_int32, ctypes.c_void_p]
    lib.rssm_materialize_checkpoints.restype = ctypes.c_int
    lib.rssm_gdn_commit.argtypes = [ctypes.POINTER(RssmGdnDesc), ctypes.POINTER(RssmGdnTables), ctypes.c_void_p]
    lib.rssm_gdn_commit.restype = ctypes.c_int
    lib.rssm_ssu_decode.argtypes = [ctypes.POINTER(RssmSsuDesc), ctypes.POINTER(RssmSsuTables), ctypes.c_void_p]
    lib.rssm_ssu_decode.restype = ctypes.c_int
    lib.rssm_last_error.argtypes = []
    lib.rssm_last_error.restype = ctypes.c_char_p
    lib.rssm_materialize_launch_config.argtypes = [ctypes.POINTER(RssmDesc), ctypes.POINTER(ctypes.c_int32),
                                                   ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.rssm_materialize_launch_config.restype = ctypes.c_int
    lib.rssm_debug_encode_rows.argtypes = [ctypes.POINTER(RssmDesc), ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.c_void_p]
    lib.rssm_debug_encode_rows.restype = ctypes.c_int
    lib.rssm_debug_row_scales.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_int32, ctypes.c_void_p]
    lib.rssm_debug_row_scales.restype = ctypes.c_int
    return lib


_lib = _load()
_pool = None


def lib():
    return _lib


def pool_lib():
    """The placement helper's library (loaded on first use)."""
    global _pool
    if _pool is None:
        if not os.path.exists(POOL_LIB_PATH):
            raise ImportError(f"{POOL_LIB_PATH} is not built. Build it with "
                              "`python -m replayssm_persistent_rssm_amd.build` (or __graft_entry__.build()).")
        pl = ctypes.CDLL(POOL_LIB_PATH)
        pl.rssm_pool_alloc.argtypes = [ctypes.c_uint64, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int32)]
        pl.rssm_pool_alloc.restype = ctypes.c_int
        pl.rssm_pool_free.argtypes = [ctypes.c_void_p]
        pl.rssm_pool_free.restype = ctypes.c_int
        _pool = pl
    return _pool


def rssm_last_error() -> str:
    return _lib.rssm_last_error().decode()


def _check(status: int):
    if status != RSSM_OK:
        raise RssmError(status, rssm_last_error())


_NAMES = {"f32": RSSM_F32, "float32": RSSM_F32, "bf16": RSSM_BF16, "bfloat16": RSSM_BF16,
          "f16": RSSM_F16, "float16": RSSM_F16, "i8": RSSM_I8, "int8": RSSM_I8,
          "f8e4m3": RSSM_F8E4M3, "float8_e4m3fn": RSSM_F8E4M3}


def dtype_code(dt) -> int:
    """Library dtype code from a name ('bf16', ...), a torch dtype or a code."""
    if isinstance(dt, int):
        return dt
    if isinstance(dt, str):
        if dt not in _NAMES:
            raise ValueError(f"unsupported dtype {dt!r}")
        return _NAMES[dt]
    name = str(dt).replace("torch.", "")
    if name in _NAMES:
        return _NAMES[name]
    raise ValueError(f"unsupported dtype {dt!r}")


def _scalar(name: str, v: int) -> int:
    v = int(v)
    if not (-_INT32_MAX - 1 <= v <= _INT32_MAX):
        raise ValueError(f"{name}={v} does not fit the library's int32 parameter")
    return v


def make_desc(*, num_layers, batch, num_heads, heads_per_group, dim, dstate, max_window, ring_buffer_len,
              state_dtype, input_dtype="bf16", matrixA_dtype="f32", pad_slot_id=-1, philox_rounds=0,
              max_workgroups=0) -> RssmDesc:
    return RssmDesc(num_layers=_scalar("num_layers", num_layers), batch=_scalar("batch", batch),
                    num_heads=_scalar("num_heads", num_heads),
                    heads_per_group=_scalar("heads_per_group", heads_per_group),
                    dim=_scalar("dim", dim), dstate=_scalar("dstate", dstate),
                    max_window=_scalar("max_window", max_window),
                    ring_buffer_len=_scalar("ring_buffer_len", ring_buffer_len),
                    pad_slot_id=_scalar("pad_slot_id", pad_slot_id),
                    philox_rounds=_scalar("philox_rounds", philox_rounds),
                    state_dtype=dtype_code(state_dtype), input_dtype=dtype_code(input_dtype),
                    a_dtype=dtype_code(matrixA_dtype), max_workgroups=_scalar("max_workgroups", max_workgroups))


def _ptr(t, name: str, dtype=None, shape=None):
    """Device address of a torch tensor after host-side metadata checks."""
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _marshal(state_ptrs, state_slot_strides, x_cache_ptrs, x_cache_slot_strides, B_cache_ptrs,
             B_cache_slot_strides, dt_cache_ptrs, dt_cache_slot_strides, A_ptrs, state_scale_ptrs,
             state_scale_slot_strides, src_slots, dst_slots, ring_start, replay_prefix_len,
             active_request_indices, *, state_dtype, input_dtype, matrixA_dtype, dim: int, dstate: int,
             num_heads: int, heads_per_group: int, max_window: int, ring_buffer_len: int, pad_slot_id: int = -1,
             rand_seed=None, philox_rounds: int = 0, max_workgroups: int = 0, num_checkpoints=None):
    """Check host-visible tensor metadata and build the C descriptor and tables.
    num_checkpoints=None: dst_slots (L, B) and replay_prefix_len (B,); else
    (C, L, B) and (C, B)."""
    import torch
    L = int(state_ptrs.shape[0])
    Bsz = int(ring_start.shape[0])
    C = () if num_checkpoints is None else (int(num_checkpoints),)
    desc = make_desc(num_layers=L, batch=Bsz, num_heads=num_heads, heads_per_group=heads_per_group, dim=dim,
                     dstate=dstate, max_window=max_window, ring_buffer_len=ring_buffer_len,
                     state_dtype=state_dtype, input_dtype=input_dtype, matrixA_dtype=matrixA_dtype,
                     pad_slot_id=pad_slot_id, philox_rounds=philox_rounds, max_workgroups=max_workgroups)
    i64, i32 = torch.int64, torch.int32
    quant = desc.state_dtype in (RSSM_I8, RSSM_F8E4M3)
    tab = RssmTables(
        state_ptrs=_ptr(state_ptrs, "state_ptrs", i64, (L,)),
        state_slot_strides=_ptr(state_slot_strides, "state_slot_strides", i64, (L,)),
        x_ptrs=_ptr(x_cache_ptrs, "x_cache_ptrs", i64, (L,)),
        x_slot_strides=_ptr(x_cache_slot_strides, "x_cache_slot_strides", i64, (L,)),
        B_ptrs=_ptr(B_cache_ptrs, "B_cache_ptrs", i64, (L,)),
        B_slot_strides=_ptr(B_cache_slot_strides, "B_cache_slot_strides", i64, (L,)),
        dt_ptrs=_ptr(dt_cache_ptrs, "dt_cache_ptrs", i64, (L,)),
        dt_slot_strides=_ptr(dt_cache_slot_strides, "dt_cache_slot_strides", i64, (L,)),
        A_ptrs=_ptr(A_ptrs, "A_ptrs", i64, (L,)),
        scale_ptrs=_ptr(state_scale_ptrs, "state_scale_ptrs", i64, (L,))
        if quant or state_scale_ptrs is not None else None,
        scale_slot_strides=_ptr(state_scale_slot_strides, "state_scale_slot_strides", i64, (L,))
        if quant or state_scale_slot_strides is not None else None,
        src_slots=_ptr(src_slots, "src_slots", i32, (L, Bsz)),
        dst_slots=_ptr(dst_slots, "dst_slots", i32, C + (L, Bsz)),
        ring_start=_ptr(ring_start, "ring_start", i32, (Bsz,)),
        replay_prefix_len=_ptr(replay_prefix_len, "replay_prefix_len", i32, C + (Bsz,)),
        active_request_indices=_ptr(active_request_indices, "active_request_indices", i32, (Bsz,)),
        rand_seed=_ptr(rand_seed, "rand_seed", i64, (1,)) if rand_seed is not None else None)
    return desc, tab


def rssm_materialize(*args, stream=None, **kw) -> None:
    """Enqueue one materialize call.

    Positional arguments, in the page's order: state_ptrs, state_slot_strides,
    x_cache_ptrs, x_cache_slot_strides, B_cache_ptrs, B_cache_slot_strides,
    dt_cache_ptrs, dt_cache_slot_strides, A_ptrs, state_scale_ptrs,
    state_scale_slot_strides, src_slots, dst_slots, ring_start,
    replay_prefix_len, active_request_indices.  Keywords: state_dtype,
    input_dtype, matrixA_dtype, dim, dstate, num_heads, heads_per_group,
    max_window, ring_buffer_len, pad_slot_id=-1, rand_seed=None,
    philox_rounds=0, max_workgroups=0.

    Per-layer tables are device int64 tensors of shape (L,); src_slots and
    dst_slots device int32 (L, B); ring_start, replay_prefix_len and
    active_request_indices device int32 (B,); rand_seed a device int64 (1,)
    tensor.  Enqueued on `stream` (default: torch's current stream)."""
    desc, tab = _marshal(*args, **kw)
    _check(_lib.rssm_materialize(ctypes.byref(desc), ctypes.byref(tab), _stream_handle(stream)))


# The page's name for the same call.
replayssm_materialize = rssm_materialize


def _num_checkpoints(dst_slots) -> int:
    if getattr(dst_slots, "dim", lambda: 0)() != 3:
        raise ValueError("dst_slots of a multi-checkpoint call has shape (num_checkpoints, L, B)")
    return int(dst_slots.shape[0])


def rssm_materialize_checkpoints(*args, stream=None, **kw) -> None:
    """Enqueue one multi-checkpoint call: the arguments of rssm_materialize,
    except that dst_slots is a device int32 (C, L, B) tensor and
    replay_prefix_len a device int32 (C, B) tensor, C in [1, 4] checkpoints
    per request (C is dst_slots.shape[0])."""
    C = _num_checkpoints(args[12] if len(args) > 12 else kw["dst_slots"])
    desc, tab = _marshal(*args, num_checkpoints=C, **kw)
    _check(_lib.rssm_materialize_checkpoints(ctypes.byref(desc), ctypes.byref(tab), C, _stream_handle(stream)))


class MaterializeCall:
    """A prepared rssm_materialize (or, with checkpoints=True,
    rssm_materialize_checkpoints): the arguments are checked and marshalled
    once, and each call is one C call with the stored descriptor and tables.

    Same arguments as the entry point; stream=None binds torch's current
    stream at construction.  The object holds references to every argument
    (the tables store only device addresses), so their memory stays
    allocated while it lives.  A call may pass another device int32 tensor
    of shape (B,) as the active list; it is held until the next call that
    passes one."""

    def __init__(self, *args, stream=None, checkpoints: bool = False, **kw):
        self._ncp = None
        if checkpoints:
            self._ncp = _num_checkpoints(args[12] if len(args) > 12 else kw["dst_slots"])
        self._keep = (args, kw)
        self._active = None
        self._desc, self._tab = _marshal(*args, num_checkpoints=self._ncp, **kw)
        self._desc_ref = ctypes.byref(self._desc)
        self._tab_ref = ctypes.byref(self._tab)
        self._stream = _stream_handle(stream)
        self._batch = int(self._desc.batch)
        if self._ncp is None:
            fn = _lib.rssm_materialize
            self._call = lambda: fn(self._desc_ref, self._tab_ref, self._stream)
        else:
            fn, ncp = _lib.rssm_materialize_checkpoints, self._ncp
            self._call = lambda: fn(self._desc_ref, self._tab_ref, ncp, self._stream)

    def __call__(self, active_request_indices=None) -> None:
        if active_request_indices is not None:
            import torch
            self._tab.active_request_indices = _ptr(active_request_indices, "active_request_indices",
                                                    torch.int32, (self._batch,))
            self._active = active_request_indices
        st = self._call()
        if st != RSSM_OK:
            raise RssmError(st, rssm_last_error())


def _gdn_marshal(checkpoint_state, rawv_cache, rawk_cache, g_cache, beta_cache, state_indices, accept_lens, *,
                 track_state_indices=None, track_steps=None, use_qk_l2norm: bool = True, null_block_id: int = -1,
                 max_workgroups: int = 0):
    import torch
    if checkpoint_state.dim() != 5 or tuple(checkpoint_state.shape[3:]) != (128, 128):
        raise ValueError("checkpoint_state must be [layers, slots, HV, 128, 128]")
    L, S, HV = (int(v) for v in checkpoint_state.shape[:3])
    if rawv_cache.dim() != 5 or rawk_cache.dim() != 5:
        raise ValueError("rawv_cache and rawk_cache must be 5-D [layers, slots, heads, T, 128]")
    T = int(rawv_cache.shape[3])
    H = int(rawk_cache.shape[2])
    B = int(state_indices.shape[0])
    if (track_state_indices is None) != (track_steps is None):
        raise ValueError("track_state_indices and track_steps go together")
    f32, bf16, i32 = torch.float32, torch.bfloat16, torch.int32
    desc = RssmGdnDesc(num_layers=_scalar("num_layers", L), slots=_scalar("slots", S), num_v_heads=_scalar("HV", HV),
                       num_k_heads=_scalar("H", H), window=_scalar("T", T), batch=_scalar("batch", B),
                       use_l2norm=1 if use_qk_l2norm else 0, null_block_id=_scalar("null_block_id", null_block_id),
                       max_workgroups=_scalar("max_workgroups", max_workgroups))
    tab = RssmGdnTables(
        checkpoint_state=_ptr(checkpoint_state, "checkpoint_state", f32, (L, S, HV, 128, 128)),
        rawv_cache=_ptr(rawv_cache, "rawv_cache", bf16, (L, S, HV, T, 128)),
        rawk_cache=_ptr(rawk_cache, "rawk_cache", bf16, (L, S, H, T, 128)),
        g_cache=_ptr(g_cache, "g_cache", f32, (L, S, HV, T)),
        beta_cache=_ptr(beta_cache, "beta_cache", f32, (L, S, HV, T)),
        state_indices=_ptr(state_indices, "state_indices", i32, (B,)),
        accept_lens=_ptr(accept_lens, "accept_lens", i32, (B,)),
        track_state_indices=_ptr(track_state_indices, "track_state_indices", i32, (B,)),
        track_steps=_ptr(track_steps, "track_steps", i32, (B,)))
    return desc, tab


def rssm_gdn_commit(*args, stream=None, **kw) -> None:
    """Enqueue one gated-delta-rule commit (the page's
    gated_delta_rule_replayssm_commit): checkpoint_state fp32 [L, slots, HV,
    128, 128] updated in place; rawv_cache bf16 [L, slots, HV, T, 128];
    rawk_cache bf16 [L, slots, H, T, 128]; g_cache and beta_cache fp32 [L,
    slots, HV, T]; state_indices and accept_lens int32 [B].  Keywords:
    track_state_indices / track_steps (int32 [B], both or neither),
    use_qk_l2norm=True, null_block_id=-1, max_workgroups=0."""
    desc, tab = _gdn_marshal(*args, **kw)
    _check(_lib.rssm_gdn_commit(ctypes.byref(desc), ctypes.byref(tab), _stream_handle(stream)))


# The page's name for the same call.
gated_delta_rule_replayssm_commit = rssm_gdn_commit


class GdnCommitCall:
    """A prepared rssm_gdn_commit: arguments checked and marshalled once; each
    call is one C call.  stream=None binds torch's current stream.  The
    object holds references to every argument (the tables store only device
    addresses), so their memory stays allocated while it lives."""

    def __init__(self, *args, stream=None, **kw):
        self._keep = (args, kw)
        self._desc, self._tab = _gdn_marshal(*args, **kw)
        self._refs = (ctypes.byref(self._desc), ctypes.byref(self._tab))
        self._stream = _stream_handle(stream)

    def __call__(self) -> None:
        st = _lib.rssm_gdn_commit(self._refs[0], self._refs[1], self._stream)
        if st != RSSM_OK:
            raise RssmError(st, rssm_last_error())


def _slot_stride(t, name: str, slots: int) -> int:
    if t.dim() < 2 or int(t.shape[0]) != slots:
        raise ValueError(f"{name} must be a pool with one row per slot ({slots} slots; got shape {tuple(t.shape)})")
    return t.numel() // slots


def _ssu_marshal(state, x_ring, B_ring, dt_ring, A, x_new, B_new, C_new, dt_new, y, slots, ring_start,
                 num_buffered, *, ring_buffer_len: int, D=None, dt_bias=None, z=None, dt_softplus: bool = True,
                 pad_slot_id: int = -1, max_workgroups: int = 0):
    import torch
    if x_new.dim() != 4 or C_new.dim() != 4:
        raise ValueError("x_new must be [B, T, H, dim] and C_new [B, T, G, dstate]")
    B, T, H, dim = (int(v) for v in x_new.shape)
    G, dstate = int(C_new.shape[2]), int(C_new.shape[3])
    if G < 1 or H % G != 0:
        raise ValueError(f"the group count of C_new ({G}) must divide the head count ({H})")
    S = int(state.shape[0])
    f32, i32, idt = torch.float32, torch.int32, x_new.dtype
    desc = RssmSsuDesc(
        batch=_scalar("batch", B), num_heads=_scalar("num_heads", H), heads_per_group=_scalar("hpg", H // G),
        dim=_scalar("dim", dim), dstate=_scalar("dstate", dstate),
        ring_buffer_len=_scalar("ring_buffer_len", ring_buffer_len), tokens=_scalar("tokens", T),
        num_slots=_scalar("num_slots", S), pad_slot_id=_scalar("pad_slot_id", pad_slot_id),
        state_dtype=dtype_code(state.dtype), input_dtype=dtype_code(idt), dt_softplus=1 if dt_softplus else 0,
        max_workgroups=_scalar("max_workgroups", max_workgroups),
        state_slot_stride=_slot_stride(state, "state", S), x_slot_stride=_slot_stride(x_ring, "x_ring", S),
        B_slot_stride=_slot_stride(B_ring, "B_ring", S), dt_slot_stride=_slot_stride(dt_ring, "dt_ring", S))
    tab = RssmSsuTables(
        state=_ptr(state, "state"), x_ring=_ptr(x_ring, "x_ring", idt), B_ring=_ptr(B_ring, "B_ring", idt),
        dt_ring=_ptr(dt_ring, "dt_ring", f32), A=_ptr(A, "A", f32, (H,)), D=_ptr(D, "D", f32, (H,)),
        dt_bias=_ptr(dt_bias, "dt_bias", f32, (H,)), x_new=_ptr(x_new, "x_new", idt),
        B_new=_ptr(B_new, "B_new", idt, (B, T, G, dstate)), C_new=_ptr(C_new, "C_new", idt),
        dt_new=_ptr(dt_new, "dt_new", f32, (B, T, H)), z=_ptr(z, "z", idt, (B, T, H, dim)),
        y=_ptr(y, "y", f32, (B, T, H, dim)), slots=_ptr(slots, "slots", i32, (B,)),
        ring_start=_ptr(ring_start, "ring_start", i32, (B,)), num_buffered=_ptr(num_buffered, "num_buffered", i32, (B,)))
    return desc, tab


def rssm_ssu_decode(*args, stream=None, **kw) -> None:
    """Enqueue one ReplaySSM decode step (one layer): the outputs y (fp32 [B,
    T, H, dim]) of T new tokens read from checkpoint + ring + the new tokens,
    which are appended to the ring; the checkpoint is not written.
    Positional: state pool [slots, ...] (f32/bf16/f16), x_ring / B_ring pools
    [slots, ...] (input dtype), dt_ring pool [slots, ...] fp32, A fp32 [H],
    x_new [B, T, H, dim], B_new / C_new [B, T, G, dstate], dt_new fp32 [B, T,
    H] (raw), y, slots / ring_start / num_buffered int32 [B].  Pools are
    contiguous with one row per slot; the slot stride is the row size.
    Keywords: ring_buffer_len (required), D, dt_bias, z (optional),
    dt_softplus=True, pad_slot_id=-1, max_workgroups=0."""
    desc, tab = _ssu_marshal(*args, **kw)
    _check(_lib.rssm_ssu_decode(ctypes.byref(desc), ctypes.byref(tab), _stream_handle(stream)))


class SsuDecodeCall:
    """A prepared rssm_ssu_decode: arguments checked and marshalled once; each
    call is one C call.  stream=None binds torch's current stream.  The
    object holds references to every argument (the tables store only device
    addresses), so their memory stays allocated while it lives."""

    def __init__(self, *args, stream=None, **kw):
        self._keep = (args, kw)
        self._desc, self._tab = _ssu_marshal(*args, **kw)
        self._refs = (ctypes.byref(self._desc), ctypes.byref(self._tab))
        self._stream = _stream_handle(stream)

    def __call__(self) -> None:
        st = _lib.rssm_ssu_decode(self._refs[0], self._refs[1], self._stream)
        if st != RSSM_OK:
            raise RssmError(st, rssm_last_error())


def rssm_pool_alloc(nbytes: int):
    """(address, contiguous) of `nbytes` of device memory on the current
    device, physically contiguous when possible (rssm_pool.h)."""
    out, contig = ctypes.c_void_p(), ctypes.c_int32()
    st = pool_lib().rssm_pool_alloc(ctypes.c_uint64(int(nbytes)), ctypes.byref(out), ctypes.byref(contig))
    if st != RSSM_OK:
        raise RssmError(st, "rssm_pool_alloc failed" if st == RSSM_ERR_HIP else "invalid size")
    return out.value, bool(contig.value)


def rssm_pool_free(addr) -> None:
    st = pool_lib().rssm_pool_free(ctypes.c_void_p(addr))
    if st != RSSM_OK:
        raise RssmError(st, "rssm_pool_free failed")


def use_contiguous_allocator() -> None:
    """Route every torch device allocation of this process through the
    contiguous pool allocator of librssm_pool (rssm_torch_pool_alloc /
    rssm_torch_pool_free; no caching: each free waits for the device).  Must
    run before the process allocates any device memory.  On MI355X a large
    pool from a plain allocation can stream markedly slower (rssm_pool.h)."""
    import torch
    pool_lib()   # fails loudly if the helper library is not built
    alloc = torch.cuda.memory.CUDAPluggableAllocator(POOL_LIB_PATH, "rssm_torch_pool_alloc", "rssm_torch_pool_free")
    torch.cuda.memory.change_current_allocator(alloc)


def rssm_materialize_launch_config(**desc_kw):
    """(grid, block, lds_bytes) the library would launch for these scalars."""
    desc = make_desc(**desc_kw)
    g, b, s = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.rssm_materialize_launch_config(ctypes.byref(desc), ctypes.byref(g), ctypes.byref(b),
                                               ctypes.byref(s)))
    return g.value, b.value, s.value


def rssm_debug_encode_rows(rows, coords, rand_seed, out_codes, out_scales, *, state_dtype, dstate: int,
                           philox_rounds: int = 0, stream=None) -> None:
    """Run the kernel's encode step on fp32 rows [n, dstate] (test hook)."""
    import torch
    n = int(rows.shape[0])
    desc = make_desc(num_layers=1, batch=1, num_heads=1, heads_per_group=1, dim=64, dstate=dstate,
                     max_window=1, ring_buffer_len=1, state_dtype=state_dtype, philox_rounds=philox_rounds)
    _check(_lib.rssm_debug_encode_rows(
        ctypes.byref(desc), _ptr(rows, "rows", torch.float32, (n, dstate)),
        _ptr(coords, "coords", torch.int32, (n, 4)) if coords is not None else None,
        _ptr(rand_seed, "rand_seed", torch.int64, (1,)) if rand_seed is not None else None,
        _ptr(out_codes, "out_codes"), _ptr(out_scales, "out_scales") if out_scales is not None else None,
        n, _stream_handle(stream)))


def rssm_debug_row_scales(rowmax, scale, inv, *, state_dtype, stream=None) -> None:
    """Row scale and inverse scale of the one-byte encode for row maxima [n] (test hook)."""
    import torch
    n = int(rowmax.shape[0])
    _check(_lib.rssm_debug_row_scales(
        dtype_code(state_dtype), _ptr(rowmax, "rowmax", torch.float32, (n,)),
        _ptr(scale, "scale", torch.float32, (n,)), _ptr(inv, "inv", torch.float32, (n,)), n,
        _stream_handle(stream)))


def pointer_table(tensors: Sequence, device) -> "torch.Tensor":
    """Device int64 table of the base addresses of per-layer tensors."""
    import torch
    return torch.tensor([int(t.data_ptr()) for t in tensors], dtype=torch.int64, device=device)


def stride_table(strides: Sequence[int], device) -> "torch.Tensor":
    import torch
    return torch.tensor([int(s) for s in strides], dtype=torch.int64, device=device)


def checkpoint_prefix_len(materialized_pos: int, buffered: int, period: int) -> Optional[int]:
    """replay_prefix_len a prefix cache passes to write its next checkpoint.

    The source state is the state after token `materialized_pos`; the ring
    holds `buffered` further accepted tokens; checkpoints are kept every
    `period` tokens.  Returns the number of ring entries up to the next
    multiple of `period`, or None when the ring does not reach it (caller
    policy from the materialize documentation's Notes and the pull request's
    Description; the kernel itself has no such logic)."""
    if period <= 0 or buffered < 0 or materialized_pos < 0:
        raise ValueError("period must be > 0; positions and counts >= 0")
    to_boundary = period - (materialized_pos % period)
    return to_boundary if to_boundary <= buffered else None

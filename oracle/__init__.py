"""CPU oracle for ReplaySSM prefix materialize -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It marshals numpy arrays into the plain C oracle
(``rssm_oracle.c``); every step of the arithmetic is there.  It imports
nothing from the HIP path; inputs come from ``rssm_inputs``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librssm_oracle.so")
SRC_PATH = os.path.join(_HERE, "rssm_oracle.c")
GDN_SRC_PATH = os.path.join(_HERE, "gdn_oracle.c")
SSU_SRC_PATH = os.path.join(_HERE, "ssu_oracle.c")

DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2, "i8": 3, "f8e4m3": 4, "f64": 5}
ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "i8": 1, "f8e4m3": 1, "f64": 8}
STORAGE_NP = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16,
              "i8": np.int8, "f8e4m3": np.uint8, "f64": np.float64}


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (IEEE arithmetic: no fast-math, no contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", SRC_PATH, GDN_SRC_PATH, SSU_SRC_PATH, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class _Params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_layers", "batch", "num_heads", "heads_per_group", "dim", "dstate", "max_window",
        "ring_len", "pad_slot_id", "philox_rounds", "state_dtype", "input_dtype")] + [
        ("seed", ctypes.c_uint64)]


_VP = ctypes.c_void_p
_P = ctypes.POINTER


class _Inputs(ctypes.Structure):
    _fields_ = [("state", _P(_VP)), ("state_stride", _P(ctypes.c_int64)),
                ("scale", _P(_VP)), ("scale_stride", _P(ctypes.c_int64)),
                ("x", _P(_VP)), ("x_stride", _P(ctypes.c_int64)),
                ("Bm", _P(_VP)), ("B_stride", _P(ctypes.c_int64)),
                ("dt", _P(_VP)), ("dt_stride", _P(ctypes.c_int64)),
                ("A", _P(_VP)),
                ("src_slots", _P(ctypes.c_int32)), ("dst_slots", _P(ctypes.c_int32)),
                ("ring_start", _P(ctypes.c_int32)), ("prefix_len", _P(ctypes.c_int32)),
                ("active", _P(ctypes.c_int32))]


class _Outputs(ctypes.Structure):
    _fields_ = [("state", _P(_VP)), ("scale", _P(_VP)), ("exact", _P(_VP)), ("mag", _P(_VP))]


class _GdnParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_layers", "slots", "num_v_heads", "num_k_heads", "window", "batch", "dk", "dv", "use_l2norm",
        "null_block_id", "has_track")]


class _GdnInputs(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("state", "rawv", "rawk", "g", "beta", "state_indices", "accept_lens",
                                    "track_state_indices", "track_steps")]


class _GdnOutputs(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("state_out", "exact", "mag")]


class _SsuParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_heads", "heads_per_group", "dim", "dstate", "ring_len", "tokens", "pad_slot_id",
        "state_dtype", "input_dtype", "dt_softplus")]


class _SsuInputs(ctypes.Structure):
    _fields_ = [("state", _VP), ("state_stride", ctypes.c_int64), ("x_ring", _VP), ("x_stride", ctypes.c_int64),
                ("B_ring", _VP), ("B_stride", ctypes.c_int64), ("dt_ring", _VP), ("dt_stride", ctypes.c_int64),
                ("A", _VP), ("D", _VP), ("dt_bias", _VP), ("x_new", _VP), ("B_new", _VP), ("C_new", _VP),
                ("dt_new", _VP), ("z", _VP), ("slots", _VP), ("ring_start", _VP), ("num_buffered", _VP)]


class _SsuOutputs(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("x_ring", "B_ring", "dt_ring", "y", "ymag", "dt_exact")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.orc_materialize.argtypes = [_P(_Params), _P(_Inputs), _P(_Outputs)]
        L.orc_materialize.restype = ctypes.c_int
        L.orc_tile.argtypes = [_P(_Params), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                               ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                               _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
        L.orc_tile.restype = ctypes.c_int
        L.orc_encode_row.argtypes = [_P(_Params), _VP, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, _VP, _VP]
        L.orc_encode_row.restype = ctypes.c_int
        L.orc_round_value.argtypes = [ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_uint32]
        L.orc_round_value.restype = ctypes.c_uint32
        L.orc_decode.argtypes = [ctypes.c_int32, _VP, ctypes.c_int64]
        L.orc_decode.restype = ctypes.c_double
        L.orc_philox4x32.argtypes = [_P(ctypes.c_uint32), _P(ctypes.c_uint32), ctypes.c_int32,
                                     _P(ctypes.c_uint32)]
        L.orc_philox4x32.restype = None
        L.orc_gdn_commit.argtypes = [_P(_GdnParams), _P(_GdnInputs), _P(_GdnOutputs)]
        L.orc_gdn_commit.restype = ctypes.c_int
        L.orc_gdn_tile.argtypes = [_P(_GdnParams), _VP, _VP, _VP, _VP, _VP, ctypes.c_int32, ctypes.c_int32,
                                   _VP, _VP, _VP, _VP]
        L.orc_gdn_tile.restype = ctypes.c_int
        L.orc_ssu_decode.argtypes = [_P(_SsuParams), _P(_SsuInputs), _P(_SsuOutputs)]
        L.orc_ssu_decode.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle buffers must be C-contiguous"
    return a.ctypes.data_as(_VP)


def _ptr_array(arrs):
    return (_VP * len(arrs))(*[a.ctypes.data for a in arrs])


def _i64(vals):
    return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


def _i32p(a: np.ndarray):
    return np.ascontiguousarray(a, np.int32).ctypes.data_as(_P(ctypes.c_int32))


def params(spec, state_dtype: Optional[str] = None, philox_rounds: Optional[int] = None,
           seed: Optional[int] = None) -> _Params:
    rounds = spec.philox_rounds if philox_rounds is None else philox_rounds
    sd = spec.rand_seed if seed is None else seed
    return _Params(num_layers=spec.L, batch=spec.B, num_heads=spec.H, heads_per_group=spec.hpg,
                   dim=spec.dim, dstate=spec.dstate, max_window=spec.W, ring_len=spec.R,
                   pad_slot_id=spec.pad_slot_id, philox_rounds=rounds,
                   state_dtype=DTYPE_CODE[state_dtype or spec.state_dtype],
                   input_dtype=DTYPE_CODE[spec.input_dtype],
                   seed=(int(sd) if sd is not None else 0) & 0xFFFFFFFFFFFFFFFF)


class OracleError(RuntimeError):
    pass


def materialize(prob, want_exact: bool = False, state_dtype: Optional[str] = None,
                philox_rounds: Optional[int] = None, seed: Optional[int] = None):
    """Run the whole operation on a host problem (``rssm_inputs.Problem``).

    Returns (state_out, scale_out, exact, mag): per-layer copies of the state
    (and scale) pools with the destination tiles written, and -- when
    ``want_exact`` -- per-layer fp64 pools holding the unrounded result and the
    magnitude sum of every written element (NaN elsewhere)."""
    return materialize_checkpoints(prob, [prob.meta.dst], [prob.meta.prefix], want_exact,
                                   state_dtype, philox_rounds, seed)


def materialize_checkpoints(prob, dst_list, prefix_list, want_exact: bool = False,
                            state_dtype: Optional[str] = None, philox_rounds: Optional[int] = None,
                            seed: Optional[int] = None):
    """Several checkpoints per request in one operation: checkpoint c writes,
    for every selected (layer, request), the state after prefix_list[c][b]
    ring entries to slot dst_list[c][l, b].  By definition each checkpoint is
    the single-checkpoint materialize with that destination table and prefix
    table, and every checkpoint reads the state and ring as they were before
    the operation -- so a destination may be the request's own source slot (an
    in-place flush: the pull-request page's "flush" of the buffered tokens into
    the state), and a checkpoint whose destination is the pad slot is skipped
    on its own.  The ring-buffer scheme of the flashinfer pages keeps several
    states per request (the gated-delta-rule commit page's track_steps writes
    an extra checkpoint next to the in-place commit).

    Returns (state_out, scale_out, exact, mag) as ``materialize``."""
    spec, meta = prob.spec, prob.meta
    if len(dst_list) != len(prefix_list) or not dst_list:
        raise ValueError("one prefix table per destination table, at least one")
    sdt = state_dtype or spec.state_dtype
    p = params(spec, sdt, philox_rounds, seed)
    src_arr = np.ascontiguousarray(meta.src, np.int32)
    rs = np.ascontiguousarray(meta.ring_start, np.int32)
    ac = np.ascontiguousarray(meta.active, np.int32)
    # the pre-call snapshot every checkpoint reads
    state_in = [np.ascontiguousarray(s).copy() for s in prob.state]
    scale_in = [np.ascontiguousarray(s).copy() for s in prob.scale] if prob.scale else None
    state_out = [s.copy() for s in state_in]
    scale_out = [s.copy() for s in scale_in] if scale_in else None
    exact = mag = None
    if want_exact or sdt == "f64":
        exact = [np.full(s.shape, np.nan, np.float64) for s in state_in]
        mag = [np.full(s.shape, np.nan, np.float64) for s in state_in]
    outs = _Outputs(state=_ptr_array(state_out),
                    scale=_ptr_array(scale_out) if scale_out else None,
                    exact=_ptr_array(exact) if exact else None,
                    mag=_ptr_array(mag) if mag else None)
    for dst, pref in zip(dst_list, prefix_list):
        dst_arr = np.ascontiguousarray(dst, np.int32)
        pf = np.ascontiguousarray(pref, np.int32)
        if dst_arr.shape != src_arr.shape or pf.shape != rs.shape:
            raise ValueError("destination tables are (L, B), prefix tables (B,)")
        keep = [state_in, scale_in, prob.x, prob.Bm, prob.dt, prob.A, dst_arr, pf]
        ins = _Inputs(state=_ptr_array(state_in), state_stride=_i64(meta.state_stride),
                      scale=_ptr_array(scale_in) if scale_in else None,
                      scale_stride=_i64(meta.scale_stride),
                      x=_ptr_array(prob.x), x_stride=_i64(meta.x_stride),
                      Bm=_ptr_array(prob.Bm), B_stride=_i64(meta.B_stride),
                      dt=_ptr_array(prob.dt), dt_stride=_i64(meta.dt_stride),
                      A=_ptr_array(prob.A),
                      src_slots=src_arr.ctypes.data_as(_P(ctypes.c_int32)),
                      dst_slots=dst_arr.ctypes.data_as(_P(ctypes.c_int32)),
                      ring_start=rs.ctypes.data_as(_P(ctypes.c_int32)),
                      prefix_len=pf.ctypes.data_as(_P(ctypes.c_int32)),
                      active=ac.ctypes.data_as(_P(ctypes.c_int32)))
        st = lib().orc_materialize(ctypes.byref(p), ctypes.byref(ins), ctypes.byref(outs))
        del keep
        if st != 0:
            raise OracleError(f"orc_materialize returned {st}")
    return state_out, scale_out, exact, mag


def tile(spec, layer: int, request: int, head: int, ring_start: int, k: int, A_h: float,
         src_tile: np.ndarray, src_scale: Optional[np.ndarray], x_slot: np.ndarray,
         B_slot: np.ndarray, dt_slot: np.ndarray, want_codes: bool = True):
    """One (layer, request, head) tile.  Arrays are the dense per-slot views of
    the source slot.  Returns (codes, scale, exact, mag)."""
    p = params(spec)
    n = spec.dim * spec.dstate
    src_tile = np.ascontiguousarray(src_tile).reshape(-1)
    exact = np.empty(n, np.float64)
    mag = np.empty(n, np.float64)
    codes = np.empty(n, STORAGE_NP[spec.state_dtype]) if want_codes else None
    scale = np.empty(spec.dim, np.float32) if src_scale is not None else None
    args = [np.ascontiguousarray(a) if a is not None else None
            for a in (src_scale, x_slot, B_slot, dt_slot)]
    st = lib().orc_tile(ctypes.byref(p), layer, request, head, ring_start, k, float(A_h),
                        _ptr(src_tile), _ptr(args[0]), _ptr(args[1]), _ptr(args[2]), _ptr(args[3]),
                        _ptr(exact), _ptr(mag), _ptr(codes), _ptr(scale))
    if st != 0:
        raise OracleError(f"orc_tile returned {st}")
    return codes, scale, exact, mag


def encode_row(spec, row: np.ndarray, layer: int, request: int, head: int, r: int,
               state_dtype: Optional[str] = None, philox_rounds: Optional[int] = None,
               seed: Optional[int] = None):
    """Encode one fp32 row (length dstate) into the state dtype."""
    sdt = state_dtype or spec.state_dtype
    p = params(spec, sdt, philox_rounds, seed)
    row = np.ascontiguousarray(row, np.float32)
    assert row.shape == (spec.dstate,)
    codes = np.empty(spec.dstate, STORAGE_NP[sdt])
    scale = np.zeros(1, np.float32)
    st = lib().orc_encode_row(ctypes.byref(p), _ptr(row), layer, request, head, r, _ptr(codes), _ptr(scale))
    if st != 0:
        raise OracleError(f"orc_encode_row returned {st}")
    return codes, float(scale[0])


def round_value(dtype: str, v: float, stochastic: bool = False, u: int = 0) -> int:
    return int(lib().orc_round_value(DTYPE_CODE[dtype], float(v), 1 if stochastic else 0, int(u) & 0xFFFFFFFF))


def decode(dtype: str, codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes).reshape(-1)
    want = np.dtype(STORAGE_NP[dtype])
    if codes.dtype != want:
        if codes.dtype.itemsize != want.itemsize:
            raise ValueError(f"{dtype} codes need {want.itemsize}-byte items, got {codes.dtype}")
        codes = codes.view(want)  # reinterpret the bits, never convert values
    f = lib().orc_decode
    return np.array([f(DTYPE_CODE[dtype], _ptr(codes), i) for i in range(codes.size)], np.float64)


def philox4x32(ctr, key, rounds: int) -> np.ndarray:
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    lib().orc_philox4x32(c, k, int(rounds), o)
    return np.array(list(o), np.uint32)


# ---------------------------------------------------------------------------
# Gated-delta-rule ReplaySSM commit
# (flashinfer.gdn_decode.gated_delta_rule_replayssm_commit; see gdn_oracle.h)
# ---------------------------------------------------------------------------
def gdn_params(spec, batch: Optional[int] = None, has_track: bool = False) -> _GdnParams:
    return _GdnParams(num_layers=spec.L, slots=spec.slots, num_v_heads=spec.HV, num_k_heads=spec.H,
                      window=spec.T, batch=spec.B if batch is None else batch, dk=spec.dk, dv=spec.dv,
                      use_l2norm=1 if spec.use_l2norm else 0, null_block_id=spec.null_block_id,
                      has_track=1 if has_track else 0)


def gdn_commit(prob, want_exact: bool = False):
    """The whole commit on a host problem (``rssm_inputs.GdnProblem``).
    Returns (state_out, exact, mag): the fp32 state pool after the commit and,
    with ``want_exact``, fp64 pools of the unrounded result and the magnitude
    bound of every written tile (NaN elsewhere)."""
    spec = prob.spec
    has_track = prob.track_state_indices is not None
    p = gdn_params(spec, has_track=has_track)
    arrs = dict(state=np.ascontiguousarray(prob.state, np.float32),
                rawv=np.ascontiguousarray(prob.rawv, np.uint16), rawk=np.ascontiguousarray(prob.rawk, np.uint16),
                g=np.ascontiguousarray(prob.g, np.float32), beta=np.ascontiguousarray(prob.beta, np.float32),
                state_indices=np.ascontiguousarray(prob.state_indices, np.int32),
                accept_lens=np.ascontiguousarray(prob.accept_lens, np.int32))
    if has_track:
        arrs["track_state_indices"] = np.ascontiguousarray(prob.track_state_indices, np.int32)
        arrs["track_steps"] = np.ascontiguousarray(prob.track_steps, np.int32)
    ins = _GdnInputs(**{k: v.ctypes.data for k, v in arrs.items()})
    state_out = arrs["state"].copy()
    exact = mag = None
    if want_exact:
        exact = np.full(state_out.shape, np.nan, np.float64)
        mag = np.full(state_out.shape, np.nan, np.float64)
    outs = _GdnOutputs(state_out=state_out.ctypes.data, exact=exact.ctypes.data if exact is not None else None,
                       mag=mag.ctypes.data if mag is not None else None)
    st = lib().orc_gdn_commit(ctypes.byref(p), ctypes.byref(ins), ctypes.byref(outs))
    if st != 0:
        raise OracleError(f"orc_gdn_commit returned {st}")
    return state_out, exact, mag


def gdn_tile(spec, s0, k_win, v_win, g_win, b_win, n: int, track_step: int = -1):
    """One (layer, request, value head) tile.  Returns (final, final_mag,
    track, track_mag) in fp64; track entries are None unless
    0 <= track_step < n."""
    p = gdn_params(spec)
    a = [np.ascontiguousarray(s0, np.float32), np.ascontiguousarray(k_win, np.uint16),
         np.ascontiguousarray(v_win, np.uint16), np.ascontiguousarray(g_win, np.float32),
         np.ascontiguousarray(b_win, np.float32)]
    shape = (spec.dv, spec.dk)
    fin, finm = np.empty(shape, np.float64), np.empty(shape, np.float64)
    trk, trkm = np.empty(shape, np.float64), np.empty(shape, np.float64)
    st = lib().orc_gdn_tile(ctypes.byref(p), *[x.ctypes.data for x in a], int(n), int(track_step),
                            fin.ctypes.data, finm.ctypes.data, trk.ctypes.data, trkm.ctypes.data)
    if st != 0:
        raise OracleError(f"orc_gdn_tile returned {st}")
    if 0 <= track_step < n:
        return fin, finm, trk, trkm
    return fin, finm, None, None


# ---------------------------------------------------------------------------
# ReplaySSM decode step (one layer; see ssu_oracle.h for the readings)
# ---------------------------------------------------------------------------
def ssu_decode(prob):
    """The decode step on a host problem (``rssm_inputs.SsuProblem``).
    Returns (x_ring, B_ring, dt_ring, y, ymag, dt_exact): the layer's rings
    after the append (storage dtypes), and fp64 outputs [B, T, H, dim] with
    their magnitude bounds (NaN for padded requests) and the new tokens' fp64
    dt [B, T, H]."""
    spec, pools = prob.spec, prob.pools
    m = pools.meta
    p = _SsuParams(batch=spec.B, num_heads=spec.H, heads_per_group=spec.hpg, dim=spec.dim, dstate=spec.dstate,
                   ring_len=spec.R, tokens=spec.T, pad_slot_id=spec.pad_slot_id,
                   state_dtype=DTYPE_CODE[spec.state_dtype], input_dtype=DTYPE_CODE[spec.input_dtype],
                   dt_softplus=1 if spec.dt_softplus else 0)
    c = lambda a: np.ascontiguousarray(a) if a is not None else None  # noqa: E731
    arrs = dict(state=c(pools.state[0]), x_ring=c(pools.x[0]), B_ring=c(pools.Bm[0]), dt_ring=c(pools.dt[0]),
                A=c(prob.A), D=c(prob.D), dt_bias=c(prob.dt_bias), x_new=c(prob.x_new), B_new=c(prob.B_new),
                C_new=c(prob.C_new), dt_new=c(prob.dt_new), z=c(prob.z),
                slots=c(prob.slots.astype(np.int32)), ring_start=c(prob.ring_start.astype(np.int32)),
                num_buffered=c(prob.num_buffered.astype(np.int32)))
    ptr = lambda k: arrs[k].ctypes.data if arrs[k] is not None else None  # noqa: E731
    ins = _SsuInputs(state=ptr("state"), state_stride=int(m.state_stride[0]), x_ring=ptr("x_ring"),
                     x_stride=int(m.x_stride[0]), B_ring=ptr("B_ring"), B_stride=int(m.B_stride[0]),
                     dt_ring=ptr("dt_ring"), dt_stride=int(m.dt_stride[0]), A=ptr("A"), D=ptr("D"),
                     dt_bias=ptr("dt_bias"), x_new=ptr("x_new"), B_new=ptr("B_new"), C_new=ptr("C_new"),
                     dt_new=ptr("dt_new"), z=ptr("z"), slots=ptr("slots"), ring_start=ptr("ring_start"),
                     num_buffered=ptr("num_buffered"))
    xr, Br, dtr = arrs["x_ring"].copy(), arrs["B_ring"].copy(), arrs["dt_ring"].copy()
    shape = (spec.B, spec.T, spec.H, spec.dim)
    y = np.full(shape, np.nan, np.float64)
    ym = np.full(shape, np.nan, np.float64)
    dte = np.full((spec.B, spec.T, spec.H), np.nan, np.float64)
    outs = _SsuOutputs(x_ring=xr.ctypes.data, B_ring=Br.ctypes.data, dt_ring=dtr.ctypes.data, y=y.ctypes.data,
                       ymag=ym.ctypes.data, dt_exact=dte.ctypes.data)
    st = lib().orc_ssu_decode(ctypes.byref(p), ctypes.byref(ins), ctypes.byref(outs))
    if st != 0:
        raise OracleError(f"orc_ssu_decode returned {st}")
    return xr, Br, dtr, y, ym, dte

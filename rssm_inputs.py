"""Seeded synthetic inputs for ReplaySSM prefix materialize.

This module is the only code shared by the CPU oracle (``oracle/``) and the
HIP path (``replayssm_persistent_rssm_amd``).  It draws inputs and nothing
else: it holds none of the operation's arithmetic.  Every array is drawn from
``numpy.random.default_rng(seed)`` (host problems) or a seeded
``torch.Generator`` on the device (full-size problems that do not fit the
host), with the shapes and value distributions of the workloads below.

Value distributions (all workloads): state N(0,1); x N(0,1); B N(0, 1/dstate);
dt U(0.001, 0.1), stored after softplus; A_h = -exp(U(0, ln 16)), so A is in
[-16, -1].  One-byte state is drawn as an N(0,1) fp32 state and quantized per
(head, row) with scale = rowmax|S| / qmax (qmax 127 for int8, 448 for e4m3).

Per-slot layouts (dense inside a slot; a slot stride may add a gap):
  state [H, dim, dstate]     scale [H, dim] fp32
  x     [R, H, dim]          B     [R, G, dstate]       dt [R, H] fp32
  A     [H] fp32 per layer
The ring (x, B, dt) of a request is the one stored in its SOURCE slot.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

DTYPES = ("f32", "bf16", "f16", "i8", "f8e4m3", "f64")
DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2, "i8": 3, "f8e4m3": 4, "f64": 5}
ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "i8": 1, "f8e4m3": 1, "f64": 8}
# numpy container used for the raw storage of each dtype
STORAGE_NP = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16,
              "i8": np.int8, "f8e4m3": np.uint8, "f64": np.float64}
QMAX = {"i8": 127.0, "f8e4m3": 448.0}


def one_byte(dtype: str) -> bool:
    return dtype in ("i8", "f8e4m3")


@dataclasses.dataclass
class Spec:
    """Shape and structure of one workload."""
    name: str
    L: int
    B: int
    H: int
    hpg: int
    dim: int
    dstate: int
    R: int
    W: int
    state_dtype: str = "bf16"
    input_dtype: str = "bf16"
    n_active: Optional[int] = None          # None: all B requests active
    k_lo: int = 0                           # replay_prefix_len ~ U[k_lo, k_hi]
    k_hi: int = 8
    k0_frac: float = 0.0                    # fraction of requests forced to k = 0
    ring_start: Optional[Sequence[int]] = None   # explicit, else U[0, R)
    prefix: Optional[Sequence[int]] = None       # explicit, else drawn
    slots: int = 0                          # state slots per layer (0: 2*B)
    ring_slots: int = 0                     # ring slots per layer (0: = slots)
    slot_mode: str = "split"                # "split": src=b, dst=B+perm(b); "perm": disjoint random from pool; "fixed"
    src_fixed: Optional[Sequence[int]] = None
    dst_fixed: Optional[Sequence[int]] = None
    stride_pad: str = "none"                # "none" | "per_layer": + 64*(l+1) elements
    pad_frac: float = 0.0                   # fraction of (layer, request) pairs with a pad slot
    pad_slot_id: int = -1
    philox_rounds: int = 0
    rand_seed: Optional[int] = None
    active_order: str = "random"            # "random" | "sorted"

    @property
    def G(self) -> int:
        return self.H // self.hpg


# The five workloads: a tiny fp32 case, a mid bf16 case, the large hybrid-model
# shape (48 layers, 256 heads of 64x128, batch 256) with an active-count sweep,
# an int8 state case and an e4m3 + Philox stochastic-rounding case.
CONFIGS = {
    "tiny_f32": Spec("tiny_f32", L=1, B=2, H=4, hpg=2, dim=16, dstate=16, R=8, W=8,
                     state_dtype="f32", input_dtype="f32", ring_start=[0, 6], prefix=[0, 5],
                     slots=4, ring_slots=4, slot_mode="fixed", src_fixed=[0, 1], dst_fixed=[2, 3],
                     active_order="sorted"),
    "mid_bf16": Spec("mid_bf16", L=4, B=16, H=64, hpg=8, dim=64, dstate=128, R=16, W=8,
                     state_dtype="bf16", input_dtype="bf16", k_lo=0, k_hi=8,
                     slots=64, ring_slots=64, slot_mode="perm", stride_pad="per_layer"),
    "large_bf16": Spec("large_bf16", L=48, B=256, H=256, hpg=32, dim=64, dstate=128, R=16, W=8,
                       state_dtype="bf16", input_dtype="bf16", n_active=256, k_lo=1, k_hi=8,
                       slots=512, ring_slots=256, slot_mode="split"),
    "large_i8": Spec("large_i8", L=48, B=256, H=256, hpg=32, dim=64, dstate=128, R=16, W=8,
                     state_dtype="i8", input_dtype="f16", n_active=64, k_lo=1, k_hi=8, k0_frac=0.25,
                     slots=512, ring_slots=256, slot_mode="split"),
    "large_f8sr": Spec("large_f8sr", L=48, B=256, H=128, hpg=16, dim=64, dstate=128, R=32, W=16,
                       state_dtype="f8e4m3", input_dtype="bf16", n_active=128, k_lo=0, k_hi=16,
                       slots=512, ring_slots=256, slot_mode="split", philox_rounds=10, rand_seed=1234),
}


def with_(spec: Spec, **kw) -> Spec:
    """Copy of a spec with some fields replaced."""
    return dataclasses.replace(spec, **kw)


def scaled(spec: Spec, name: str, **kw) -> Spec:
    """A smaller workload with the same structure (for full-oracle parity)."""
    return dataclasses.replace(spec, name=name, **kw)


# --------------------------------------------------------------------------
# Metadata
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Meta:
    src: np.ndarray          # (L, B) int32
    dst: np.ndarray          # (L, B) int32
    ring_start: np.ndarray   # (B,) int32
    prefix: np.ndarray       # (B,) int32
    active: np.ndarray       # (B,) int32
    state_stride: List[int]  # elements, per layer
    scale_stride: List[int]
    x_stride: List[int]
    B_stride: List[int]
    dt_stride: List[int]
    slots: int
    ring_slots: int


def dense_sizes(spec: Spec):
    """Dense per-slot element counts: state, scale, x, B, dt."""
    return (spec.H * spec.dim * spec.dstate, spec.H * spec.dim,
            spec.R * spec.H * spec.dim, spec.R * spec.G * spec.dstate, spec.R * spec.H)


def make_meta(spec: Spec, rng: np.random.Generator, n_active: Optional[int] = None) -> Meta:
    L, B = spec.L, spec.B
    slots = spec.slots or 2 * B
    ring_slots = spec.ring_slots or slots
    n_act = B if (n_active is None and spec.n_active is None) else (spec.n_active if n_active is None else n_active)
    n_act = int(n_act)

    if spec.ring_start is not None:
        ring_start = np.asarray(spec.ring_start, np.int32)
    else:
        ring_start = rng.integers(0, spec.R, size=B).astype(np.int32)
    if spec.prefix is not None:
        prefix = np.asarray(spec.prefix, np.int32)
    else:
        prefix = rng.integers(spec.k_lo, spec.k_hi + 1, size=B).astype(np.int32)
        if spec.k0_frac > 0:
            n0 = int(round(spec.k0_frac * B))
            prefix[rng.permutation(B)[:n0]] = 0

    if spec.active_order == "sorted":
        chosen = np.arange(n_act, dtype=np.int32)
    else:
        chosen = rng.permutation(B)[:n_act].astype(np.int32)
    active = np.full(B, -1, np.int32)
    active[:n_act] = chosen

    src = np.empty((L, B), np.int32)
    dst = np.empty((L, B), np.int32)
    for l in range(L):
        if spec.slot_mode == "fixed":
            src[l] = np.asarray(spec.src_fixed, np.int32)
            dst[l] = np.asarray(spec.dst_fixed, np.int32)
        elif spec.slot_mode == "perm":
            perm = rng.permutation(slots)
            assert slots >= 2 * B and ring_slots >= slots
            src[l] = perm[:B]
            dst[l] = perm[B:2 * B]
        elif spec.slot_mode == "split":
            assert slots >= 2 * B and ring_slots >= B
            src[l] = np.arange(B)
            dst[l] = B + rng.permutation(B)
        else:
            raise ValueError(spec.slot_mode)
    if spec.pad_frac > 0:
        npad = int(round(spec.pad_frac * L * B))
        flat = rng.permutation(L * B)[:npad]
        which = rng.integers(0, 2, size=npad)
        for f, w in zip(flat, which):
            (src if w == 0 else dst)[f // B, f % B] = spec.pad_slot_id
    # Requests that are not listed carry pad slots, as a serving loop would.
    inactive = np.setdiff1d(np.arange(B), active[:n_act])
    if len(inactive) and spec.slot_mode == "split":
        src[:, inactive] = spec.pad_slot_id
        dst[:, inactive] = spec.pad_slot_id

    d_state, d_scale, d_x, d_B, d_dt = dense_sizes(spec)
    pad = [64 * (l + 1) if spec.stride_pad == "per_layer" else 0 for l in range(L)]
    return Meta(src=src, dst=dst, ring_start=ring_start, prefix=prefix, active=active,
                state_stride=[d_state + p for p in pad], scale_stride=[d_scale + p for p in pad],
                x_stride=[d_x + p for p in pad], B_stride=[d_B + p for p in pad],
                dt_stride=[d_dt + p for p in pad], slots=slots, ring_slots=ring_slots)


# --------------------------------------------------------------------------
# Host problems (numpy)
# --------------------------------------------------------------------------
def make_checkpoints(spec: Spec, meta: Meta, seed: int, n_ck: int, in_place: bool = False,
                     k0_frac: float = 0.0, pad_frac: float = 0.0, dup_frac: float = 0.0):
    """Destination and prefix tables of n_ck checkpoints per request:
    dst (n_ck, L, B) int32 and prefix (n_ck, B) int32.

    Checkpoint 0 is the problem's own (dst, prefix) -- or, with `in_place`,
    the source slot itself.  The others take distinct slots that neither the
    source nor the destination table uses, and prefix lengths ~ U[0, W];
    `k0_frac` forces some to 0, `dup_frac` copies checkpoint 0's length, and
    `pad_frac` replaces some destinations of checkpoints >= 1 with the pad
    slot.  Needs enough free slots: spec.slots >= (n_ck + 1) * B."""
    rng = np.random.default_rng(seed)
    L, B, pad = spec.L, spec.B, spec.pad_slot_id
    dst = np.empty((n_ck, L, B), np.int32)
    pre = np.empty((n_ck, B), np.int32)
    dst[0] = np.where(meta.src == pad, pad, meta.src) if in_place else meta.dst
    pre[0] = meta.prefix
    for c in range(1, n_ck):
        pre[c] = rng.integers(0, spec.W + 1, size=B)
        if k0_frac > 0:
            pre[c, rng.permutation(B)[:int(round(k0_frac * B))]] = 0
        if dup_frac > 0:
            sel = rng.permutation(B)[:int(round(dup_frac * B))]
            pre[c, sel] = pre[0, sel]
    for l in range(L):
        used = set(int(v) for v in meta.src[l]) | set(int(v) for v in meta.dst[l])
        free = np.array([v for v in rng.permutation(meta.slots) if int(v) not in used and int(v) != pad], np.int32)
        need = (n_ck - 1) * B
        if len(free) < need:
            raise ValueError(f"{n_ck} checkpoints need {need} free slots per layer, the pool has {len(free)}")
        for c in range(1, n_ck):
            dst[c, l] = free[(c - 1) * B:c * B]
        if pad_frac > 0 and n_ck > 1:
            npad = int(round(pad_frac * B))
            for c in range(1, n_ck):
                dst[c, l, rng.permutation(B)[:npad]] = pad
    return dst, pre


@dataclasses.dataclass
class Problem:
    spec: Spec
    meta: Meta
    state: List[np.ndarray]            # per layer (slots, state_stride), storage dtype
    scale: Optional[List[np.ndarray]]  # per layer (slots, scale_stride) fp32, 1-byte state only
    x: List[np.ndarray]                # per layer (ring_slots, x_stride)
    Bm: List[np.ndarray]
    dt: List[np.ndarray]               # fp32
    A: List[np.ndarray]                # (H,) fp32

    @property
    def rand_seed(self) -> Optional[int]:
        return self.spec.rand_seed


def _to_storage(vals: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values -> raw storage (library casts, nearest-even)."""
    if dtype == "f32":
        return vals.astype(np.float32)
    if dtype == "f64":
        return vals.astype(np.float64)
    if dtype == "f16":
        return vals.astype(np.float16)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "f8e4m3":
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(dtype)


def _quantized_rows(S: np.ndarray, dtype: str):
    """Per-row symmetric quantization of an fp32 state (input recipe only)."""
    qmax = np.float32(QMAX[dtype])
    rowmax = np.abs(S).max(axis=-1, keepdims=True).astype(np.float32)
    scale = (rowmax / qmax).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1))
    t = (S / safe).astype(np.float32)
    if dtype == "i8":
        codes = np.clip(np.rint(t), -127, 127).astype(np.int8)
    else:
        codes = _to_storage(np.clip(t, -448, 448), "f8e4m3")
    return codes, scale[..., 0]


def _draw_state(rng, spec: Spec, n_slots: int, stride: int):
    """State pool of one layer: every slot and gap holds drawn values."""
    dense = spec.H * spec.dim * spec.dstate
    if one_byte(spec.state_dtype):
        S = rng.standard_normal((n_slots, spec.H, spec.dim, spec.dstate), dtype=np.float32)
        codes, scale = _quantized_rows(S, spec.state_dtype)
        pool = rng.integers(-100, 100, size=(n_slots, stride)).astype(STORAGE_NP[spec.state_dtype]) \
            if spec.state_dtype == "i8" else rng.integers(0, 0x7E, size=(n_slots, stride)).astype(np.uint8)
        pool[:, :dense] = codes.reshape(n_slots, dense)
        d_scale = spec.H * spec.dim
        sstride = stride - dense + d_scale
        spool = rng.random((n_slots, sstride), dtype=np.float32)
        spool[:, :d_scale] = scale.reshape(n_slots, d_scale)
        return pool, spool
    vals = rng.standard_normal((n_slots, stride), dtype=np.float32)
    return _to_storage(vals, spec.state_dtype), None


def make_problem(spec: Spec, seed: int, n_active: Optional[int] = None) -> Problem:
    """Host (numpy) problem: every pool fully drawn, including gaps and dst slots."""
    rng = np.random.default_rng(seed)
    meta = make_meta(spec, rng, n_active)
    state, scale, xs, Bs, dts, As = [], [], [], [], [], []
    for l in range(spec.L):
        st, sc = _draw_state(rng, spec, meta.slots, meta.state_stride[l])
        state.append(st)
        if sc is not None:
            assert sc.shape[1] == meta.scale_stride[l]
            scale.append(sc)
        xv = rng.standard_normal((meta.ring_slots, meta.x_stride[l]), dtype=np.float32)
        xs.append(_to_storage(xv, spec.input_dtype))
        bv = rng.standard_normal((meta.ring_slots, meta.B_stride[l]), dtype=np.float32) / np.float32(math.sqrt(spec.dstate))
        Bs.append(_to_storage(bv, spec.input_dtype))
        dts.append(rng.uniform(0.001, 0.1, size=(meta.ring_slots, meta.dt_stride[l])).astype(np.float32))
        As.append((-np.exp(rng.uniform(0.0, math.log(16.0), size=spec.H))).astype(np.float32))
    return Problem(spec=spec, meta=meta, state=state, scale=scale if scale else None,
                   x=xs, Bm=Bs, dt=dts, A=As)


# --------------------------------------------------------------------------
# Device problems (torch), for workloads too large for host memory
# --------------------------------------------------------------------------
@dataclasses.dataclass
class DeviceProblem:
    spec: Spec
    meta: Meta
    state: list      # per layer torch tensors (slots, stride), raw storage dtype
    scale: Optional[list]
    x: list
    Bm: list
    dt: list
    A: list


def _torch_storage(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
            "i8": torch.int8, "f8e4m3": torch.uint8}[dtype]


def make_device_problem(spec: Spec, seed: int, device="cuda", n_active: Optional[int] = None,
                        fill_dst: int = 0xA5) -> DeviceProblem:
    """Device problem drawn with a seeded torch generator.  Only source slots
    (and the ring) get random values; every other slot is filled with the byte
    `fill_dst`, so that untouched slots can be recognised."""
    import torch
    rng = np.random.default_rng(seed)
    meta = make_meta(spec, rng, n_active)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    src_slots = np.unique(meta.src[meta.src != spec.pad_slot_id]) if (meta.src != spec.pad_slot_id).any() else np.zeros(0, np.int64)
    lo_src = int(src_slots.min()) if len(src_slots) else 0
    hi_src = int(src_slots.max()) + 1 if len(src_slots) else 0
    dense = spec.H * spec.dim * spec.dstate
    sdt = _torch_storage(spec.state_dtype)
    idt = _torch_storage(spec.input_dtype)
    state, scale, xs, Bs, dts, As = [], [], [], [], [], []
    for l in range(spec.L):
        st = torch.empty((meta.slots, meta.state_stride[l]), dtype=sdt, device=device)
        st.view(torch.uint8).fill_(fill_dst)
        sc = None
        if one_byte(spec.state_dtype):
            sc = torch.empty((meta.slots, meta.scale_stride[l]), dtype=torch.float32, device=device)
            sc.view(torch.uint8).fill_(fill_dst)
            qmax = QMAX[spec.state_dtype]
            # quantize one source slot range at a time to bound temporaries
            for s0 in range(lo_src, hi_src, 32):
                s1 = min(hi_src, s0 + 32)
                S = torch.randn((s1 - s0, spec.H, spec.dim, spec.dstate), generator=g, device=device,
                                dtype=torch.float32)
                rowmax = S.abs().amax(dim=-1, keepdim=True)
                sca = rowmax / qmax
                t = S / torch.where(sca > 0, sca, torch.ones_like(sca))
                if spec.state_dtype == "i8":
                    codes = torch.clamp(torch.round(t), -127, 127).to(torch.int8)
                else:
                    codes = torch.clamp(t, -448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
                st[s0:s1, :dense] = codes.reshape(s1 - s0, dense)
                sc[s0:s1, :spec.H * spec.dim] = sca.reshape(s1 - s0, spec.H * spec.dim)
                del S, rowmax, sca, t, codes
        else:
            for s0 in range(lo_src, hi_src, 64):
                s1 = min(hi_src, s0 + 64)
                st[s0:s1, :dense] = torch.randn((s1 - s0, dense), generator=g, device=device, dtype=sdt)
        state.append(st)
        if sc is not None:
            scale.append(sc)
        xs.append(torch.randn((meta.ring_slots, meta.x_stride[l]), generator=g, device=device, dtype=idt))
        Bs.append(torch.randn((meta.ring_slots, meta.B_stride[l]), generator=g, device=device,
                              dtype=torch.float32).mul_(1.0 / math.sqrt(spec.dstate)).to(idt))
        dts.append(torch.rand((meta.ring_slots, meta.dt_stride[l]), generator=g, device=device,
                              dtype=torch.float32).mul_(0.099).add_(0.001))
        As.append(-torch.exp(torch.rand((spec.H,), generator=g, device=device, dtype=torch.float32)
                             * math.log(16.0)))
    return DeviceProblem(spec=spec, meta=meta, state=state, scale=scale if scale else None,
                         x=xs, Bm=Bs, dt=dts, A=As)



# --------------------------------------------------------------------------
# Gated-delta-rule ReplaySSM commit (flashinfer.gdn_decode.
# gated_delta_rule_replayssm_commit): contiguous pools as on that page.
# --------------------------------------------------------------------------
@dataclasses.dataclass
class GdnSpec:
    """Shape and structure of one commit workload."""
    name: str
    L: int                     # layers
    B: int                     # requests
    HV: int                    # value heads
    H: int                     # key heads (divides HV)
    T: int                     # tokens per cached window
    slots: int                 # pool slots per layer
    dk: int = 128
    dv: int = 128
    use_l2norm: bool = True
    null_block_id: int = -1
    null_frac: float = 0.0     # requests whose slot is <= null_block_id
    track: bool = False
    accept: Optional[Sequence[int]] = None   # explicit accept_lens, else U[0, T]
    zero_frac: float = 0.0     # requests forced to accept 0


GDN_CONFIGS = {
    # all shapes the page fixes: fp32 128x128 K-last state, bf16 windows, T <= 8
    "gdn_small": GdnSpec("gdn_small", L=2, B=6, HV=4, H=2, T=8, slots=16, null_frac=0.2, track=True,
                         zero_frac=0.2),
    # 48 layers, 256 requests, 32 value heads over 16 key heads, 8-token windows
    "gdn_large": GdnSpec("gdn_large", L=48, B=256, HV=32, H=16, T=8, slots=512, null_frac=1 / 16, track=True,
                         zero_frac=1 / 16),
}


@dataclasses.dataclass
class GdnProblem:
    spec: GdnSpec
    state: np.ndarray                 # (L, slots, HV, dv, dk) fp32
    rawv: np.ndarray                  # (L, slots, HV, T, dv) bf16 codes (uint16)
    rawk: np.ndarray                  # (L, slots, H, T, dk) bf16 codes (uint16)
    g: np.ndarray                     # (L, slots, HV, T) fp32 log decay
    beta: np.ndarray                  # (L, slots, HV, T) fp32 in (0, 1)
    state_indices: np.ndarray         # (B,) int32
    accept_lens: np.ndarray           # (B,) int32
    track_state_indices: Optional[np.ndarray]
    track_steps: Optional[np.ndarray]


def make_gdn_meta(spec: GdnSpec, rng: np.random.Generator):
    """state_indices (distinct live slots above null_block_id, some requests
    null), accept_lens ~ U[0, T] (some forced 0), and -- with tracking --
    distinct track slots disjoint from the live ones and steps ~ U[-1, T-1]
    (so some fall outside the accepted prefix)."""
    B, nb = spec.B, spec.null_block_id
    live_pool = np.arange(nb + 1, spec.slots)
    need = B * (2 if spec.track else 1)
    if len(live_pool) < need:
        raise ValueError(f"{spec.name}: {need} slots needed above null_block_id, the pool has {len(live_pool)}")
    perm = rng.permutation(live_pool)
    idx = perm[:B].astype(np.int32)
    n_null = int(round(spec.null_frac * B))
    if n_null:
        idx[rng.permutation(B)[:n_null]] = rng.integers(-1, nb + 1, size=n_null) if nb >= 0 else -1
    if spec.accept is not None:
        acc = np.asarray(spec.accept, np.int32)
    else:
        acc = rng.integers(0, spec.T + 1, size=B).astype(np.int32)
        n0 = int(round(spec.zero_frac * B))
        if n0:
            acc[rng.permutation(B)[:n0]] = 0
    tidx = tstep = None
    if spec.track:
        tidx = perm[B:2 * B].astype(np.int32)
        tstep = rng.integers(-1, spec.T, size=B).astype(np.int32)
    return idx, acc, tidx, tstep


def _bf16_codes(vals: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(vals, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_gdn_problem(spec: GdnSpec, seed: int) -> GdnProblem:
    """Host problem, every pool fully drawn: state N(0,1); raw k, v N(0,1)
    in bf16; g ~ U(-1, 0) (decay exp(g) in (0.37, 1]); beta = sigmoid(N(0,1))."""
    rng = np.random.default_rng(seed)
    idx, acc, tidx, tstep = make_gdn_meta(spec, rng)
    L, S, HV, H, T = spec.L, spec.slots, spec.HV, spec.H, spec.T
    state = rng.standard_normal((L, S, HV, spec.dv, spec.dk), dtype=np.float32)
    rawv = _bf16_codes(rng.standard_normal((L, S, HV, T, spec.dv), dtype=np.float32))
    rawk = _bf16_codes(rng.standard_normal((L, S, H, T, spec.dk), dtype=np.float32))
    g = rng.uniform(-1.0, 0.0, size=(L, S, HV, T)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((L, S, HV, T))))).astype(np.float32)
    return GdnProblem(spec, state, rawv, rawk, g, beta, idx, acc, tidx, tstep)


@dataclasses.dataclass
class GdnDeviceProblem:
    spec: GdnSpec
    state: object      # torch fp32 (L, slots, HV, dv, dk)
    rawv: object       # torch bf16 (L, slots, HV, T, dv)
    rawk: object       # torch bf16 (L, slots, H, T, dk)
    g: object
    beta: object
    state_indices: np.ndarray
    accept_lens: np.ndarray
    track_state_indices: Optional[np.ndarray]
    track_steps: Optional[np.ndarray]


def make_gdn_device_problem(spec: GdnSpec, seed: int, device="cuda", fill: int = 0xA5) -> GdnDeviceProblem:
    """Full-size device problem from a seeded torch generator: the live and
    track slots' state, and every window, are drawn as in make_gdn_problem;
    every other state byte holds `fill`."""
    import torch
    rng = np.random.default_rng(seed)
    idx, acc, tidx, tstep = make_gdn_meta(spec, rng)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    L, S, HV, H, T = spec.L, spec.slots, spec.HV, spec.H, spec.T
    state = torch.empty((L, S, HV, spec.dv, spec.dk), dtype=torch.float32, device=device)
    state.view(torch.uint8).fill_(fill)
    live = sorted(set(int(v) for v in idx if v > spec.null_block_id))
    if live:
        sl = torch.tensor(live, device=device)
        for l in range(L):
            state[l, sl] = torch.randn((len(live), HV, spec.dv, spec.dk), generator=gen, device=device)
    rawv = torch.randn((L, S, HV, T, spec.dv), generator=gen, device=device).to(torch.bfloat16)
    rawk = torch.randn((L, S, H, T, spec.dk), generator=gen, device=device).to(torch.bfloat16)
    g = torch.rand((L, S, HV, T), generator=gen, device=device) - 1.0
    beta = torch.sigmoid(torch.randn((L, S, HV, T), generator=gen, device=device))
    return GdnDeviceProblem(spec, state, rawv, rawk, g, beta, idx, acc, tidx, tstep)


# --------------------------------------------------------------------------
# ReplaySSM decode step (one layer): the materialize pools of that layer plus
# the step's new tokens.
# --------------------------------------------------------------------------
@dataclasses.dataclass
class SsuSpec:
    """Shape and structure of one decode-step workload (one layer)."""
    name: str
    B: int
    H: int
    hpg: int
    dim: int
    dstate: int
    R: int
    T: int                       # new tokens per request
    state_dtype: str = "bf16"
    input_dtype: str = "bf16"
    has_z: bool = True
    has_D: bool = True
    has_bias: bool = True
    dt_softplus: bool = True
    slots: int = 0               # state/ring slots (0: 2 * B)
    pad_frac: float = 0.0        # requests whose slot is the pad slot
    pad_slot_id: int = -1
    buffered: Optional[Sequence[int]] = None   # explicit num_buffered, else U[0, R - T]

    @property
    def G(self) -> int:
        return self.H // self.hpg

    def pools(self) -> Spec:
        """The single-layer materialize spec whose pools this step uses."""
        return Spec(self.name + "_pools", L=1, B=self.B, H=self.H, hpg=self.hpg, dim=self.dim, dstate=self.dstate,
                    R=self.R, W=min(16, self.R), state_dtype=self.state_dtype, input_dtype=self.input_dtype,
                    slots=self.slots or 2 * self.B, ring_slots=self.slots or 2 * self.B, slot_mode="perm",
                    stride_pad="per_layer", pad_slot_id=self.pad_slot_id)


SSU_CONFIGS = {
    "ssu_small": SsuSpec("ssu_small", B=5, H=8, hpg=4, dim=64, dstate=128, R=16, T=4, pad_frac=0.2),
    # one layer of the large hybrid-model shape, speculative decode with 4 tokens per step
    "ssu_large": SsuSpec("ssu_large", B=256, H=256, hpg=32, dim=64, dstate=128, R=16, T=4),
}


@dataclasses.dataclass
class SsuProblem:
    spec: SsuSpec
    pools: Problem               # state pool and rings (layer 0)
    slots: np.ndarray            # (B,) int32 checkpoint/ring slot per request (pad: skipped)
    ring_start: np.ndarray       # (B,) int32
    num_buffered: np.ndarray     # (B,) int32
    A: np.ndarray                # (H,) fp32
    D: Optional[np.ndarray]      # (H,) fp32
    dt_bias: Optional[np.ndarray]
    x_new: np.ndarray            # (B, T, H, dim) input dtype
    B_new: np.ndarray            # (B, T, G, dstate)
    C_new: np.ndarray            # (B, T, G, dstate)
    dt_new: np.ndarray           # (B, T, H) fp32, raw
    z: Optional[np.ndarray]      # (B, T, H, dim)


def make_ssu_problem(spec: SsuSpec, seed: int) -> SsuProblem:
    """Pools as make_problem (state N(0,1), x N(0,1), B N(0,1/dstate), dt
    U(0.001, 0.1)); new tokens: x N(0,1), B and C N(0, 1/dstate), z N(0,1),
    raw dt N(0, 0.3^2) with dt_bias = softplus^-1(U(0.001, 0.1)) (so dt after
    bias and softplus stays near the ring's range), D U(0.5, 1.5);
    num_buffered U[0, R - T], ring_start U[0, R)."""
    rng = np.random.default_rng(seed)
    pools = make_problem(spec.pools(), seed)
    B, H, G, T = spec.B, spec.H, spec.G, spec.T
    slots = pools.meta.src[0].astype(np.int32).copy()
    if spec.pad_frac > 0:
        slots[rng.permutation(B)[:int(round(spec.pad_frac * B))]] = spec.pad_slot_id
    ring_start = pools.meta.ring_start.astype(np.int32).copy()
    if spec.buffered is not None:
        nb = np.asarray(spec.buffered, np.int32)
    else:
        nb = rng.integers(0, spec.R - T + 1, size=B).astype(np.int32)
    A = pools.A[0].copy()
    D = rng.uniform(0.5, 1.5, size=H).astype(np.float32) if spec.has_D else None
    bias = np.log(np.expm1(rng.uniform(0.001, 0.1, size=H))).astype(np.float32) if spec.has_bias else None
    x_new = _to_storage(rng.standard_normal((B, T, H, spec.dim), dtype=np.float32), spec.input_dtype)
    sd = np.float32(1.0 / math.sqrt(spec.dstate))
    B_new = _to_storage(rng.standard_normal((B, T, G, spec.dstate), dtype=np.float32) * sd, spec.input_dtype)
    C_new = _to_storage(rng.standard_normal((B, T, G, spec.dstate), dtype=np.float32) * sd, spec.input_dtype)
    dt_new = (rng.standard_normal((B, T, H)) * 0.3).astype(np.float32)
    z = _to_storage(rng.standard_normal((B, T, H, spec.dim), dtype=np.float32), spec.input_dtype) if spec.has_z else None
    return SsuProblem(spec, pools, slots, ring_start, nb, A, D, bias, x_new, B_new, C_new, dt_new, z)


@dataclasses.dataclass
class SsuDeviceProblem:
    """A decode-step problem in device memory (torch tensors; 16-bit float
    storage as torch.bfloat16 / torch.float16)."""
    spec: SsuSpec
    state: object            # (slots, state_stride) state dtype
    x_ring: object           # (slots, x_stride) input dtype
    B_ring: object           # (slots, B_stride)
    dt_ring: object          # (slots, dt_stride) fp32
    A: object
    D: Optional[object]
    dt_bias: Optional[object]
    x_new: object
    B_new: object
    C_new: object
    dt_new: object
    z: Optional[object]
    y: object                # (B, T, H, dim) fp32, NaN-filled
    slots: object            # (B,) int32 device
    ring_start: object
    num_buffered: object
    slots_np: np.ndarray
    ring_start_np: np.ndarray
    num_buffered_np: np.ndarray


def _torch_typed(a: np.ndarray, dtype: str, device):
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def ssu_to_device(prob: SsuProblem, device="cuda") -> SsuDeviceProblem:
    """Copy a host decode-step problem to the device, same layouts."""
    import torch
    spec, pools = prob.spec, prob.pools
    it = spec.input_dtype
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device) if a is not None else None  # noqa: E731
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)  # noqa: E731
    y = torch.full((spec.B, spec.T, spec.H, spec.dim), float("nan"), dtype=torch.float32, device=device)
    return SsuDeviceProblem(
        spec=spec, state=_torch_typed(pools.state[0], spec.state_dtype, device),
        x_ring=_torch_typed(pools.x[0], it, device), B_ring=_torch_typed(pools.Bm[0], it, device),
        dt_ring=f(pools.dt[0]), A=f(prob.A), D=f(prob.D), dt_bias=f(prob.dt_bias),
        x_new=_torch_typed(prob.x_new, it, device), B_new=_torch_typed(prob.B_new, it, device),
        C_new=_torch_typed(prob.C_new, it, device), dt_new=f(prob.dt_new),
        z=_torch_typed(prob.z, it, device) if prob.z is not None else None, y=y,
        slots=i32(prob.slots), ring_start=i32(prob.ring_start), num_buffered=i32(prob.num_buffered),
        slots_np=prob.slots.astype(np.int32), ring_start_np=prob.ring_start.astype(np.int32),
        num_buffered_np=prob.num_buffered.astype(np.int32))


def make_ssu_device_problem(spec: SsuSpec, seed: int, device="cuda") -> SsuDeviceProblem:
    """Full-size decode-step problem drawn on the device (seeded torch
    generator) with the distributions of make_ssu_problem; the pools are
    make_device_problem's (request slots random, every other slot's state
    filled with the byte 0xA5)."""
    import torch
    rng = np.random.default_rng(seed)
    pools = make_device_problem(spec.pools(), seed, device)
    B, H, G, T = spec.B, spec.H, spec.G, spec.T
    slots = pools.meta.src[0].astype(np.int32).copy()
    if spec.pad_frac > 0:
        slots[rng.permutation(B)[:int(round(spec.pad_frac * B))]] = spec.pad_slot_id
    ring_start = pools.meta.ring_start.astype(np.int32).copy()
    if spec.buffered is not None:
        nb = np.asarray(spec.buffered, np.int32)
    else:
        nb = rng.integers(0, spec.R - T + 1, size=B).astype(np.int32)
    g = torch.Generator(device=device)
    g.manual_seed(seed + 1)
    idt = _torch_storage(spec.input_dtype)
    sd = 1.0 / math.sqrt(spec.dstate)
    rn = lambda *shape: torch.randn(shape, generator=g, device=device, dtype=torch.float32)  # noqa: E731
    D = torch.from_numpy(rng.uniform(0.5, 1.5, size=H).astype(np.float32)).to(device) if spec.has_D else None
    bias = (torch.from_numpy(np.log(np.expm1(rng.uniform(0.001, 0.1, size=H))).astype(np.float32)).to(device)
            if spec.has_bias else None)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)  # noqa: E731
    y = torch.full((B, T, H, spec.dim), float("nan"), dtype=torch.float32, device=device)
    return SsuDeviceProblem(
        spec=spec, state=pools.state[0], x_ring=pools.x[0], B_ring=pools.Bm[0], dt_ring=pools.dt[0], A=pools.A[0],
        D=D, dt_bias=bias, x_new=rn(B, T, H, spec.dim).to(idt), B_new=rn(B, T, G, spec.dstate).mul_(sd).to(idt),
        C_new=rn(B, T, G, spec.dstate).mul_(sd).to(idt), dt_new=rn(B, T, H).mul_(0.3),
        z=rn(B, T, H, spec.dim).to(idt) if spec.has_z else None, y=y, slots=i32(slots), ring_start=i32(ring_start),
        num_buffered=i32(nb), slots_np=slots, ring_start_np=ring_start, num_buffered_np=nb)

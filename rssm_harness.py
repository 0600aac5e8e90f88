"""Drive librssm_materialize on the seeded workloads of ``rssm_inputs``.

Marshalling only: upload host problems to the device, build the per-layer
pointer/stride tables and metadata tensors, call the library through its
binding, download results.  Used by the GPU tests, the smoke check and the
benchmark.  It never imports the CPU oracle.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

import rssm_inputs as ri


def _np_to_dev(a: np.ndarray, device):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def upload(prob: ri.Problem, device="cuda") -> ri.DeviceProblem:
    """Copy a host problem to the device with the same per-layer layout."""
    up = lambda arrs: [_np_to_dev(x, device) for x in arrs] if arrs is not None else None  # noqa: E731
    return ri.DeviceProblem(spec=prob.spec, meta=prob.meta, state=up(prob.state), scale=up(prob.scale),
                            x=up(prob.x), Bm=up(prob.Bm), dt=up(prob.dt), A=up(prob.A))


def download(tensors, like: Optional[list] = None):
    out = []
    for i, t in enumerate(tensors):
        a = t.detach().cpu().contiguous()
        import torch
        if a.dtype == torch.bfloat16:
            a = a.view(torch.int16)
        n = a.numpy()
        if like is not None:
            n = n.view(like[i].dtype)
        elif n.dtype == np.int16:
            n = n.view(np.uint16)
        out.append(n)
    return out


@dataclasses.dataclass
class Tables:
    state_ptrs: object
    state_slot_strides: object
    x_cache_ptrs: object
    x_cache_slot_strides: object
    B_cache_ptrs: object
    B_cache_slot_strides: object
    dt_cache_ptrs: object
    dt_cache_slot_strides: object
    A_ptrs: object
    state_scale_ptrs: object
    state_scale_slot_strides: object
    src_slots: object
    dst_slots: object
    ring_start: object
    replay_prefix_len: object
    active_request_indices: object
    rand_seed: object


def tables(dp: ri.DeviceProblem, device="cuda", active: Optional[np.ndarray] = None) -> Tables:
    import torch
    from replayssm_persistent_rssm_amd import pointer_table, stride_table
    m = dp.meta
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)  # noqa: E731
    seed = dp.spec.rand_seed
    return Tables(
        state_ptrs=pointer_table(dp.state, device), state_slot_strides=stride_table(m.state_stride, device),
        x_cache_ptrs=pointer_table(dp.x, device), x_cache_slot_strides=stride_table(m.x_stride, device),
        B_cache_ptrs=pointer_table(dp.Bm, device), B_cache_slot_strides=stride_table(m.B_stride, device),
        dt_cache_ptrs=pointer_table(dp.dt, device), dt_cache_slot_strides=stride_table(m.dt_stride, device),
        A_ptrs=pointer_table(dp.A, device),
        state_scale_ptrs=pointer_table(dp.scale, device) if dp.scale else None,
        state_scale_slot_strides=stride_table(m.scale_stride, device) if dp.scale else None,
        src_slots=i32(m.src), dst_slots=i32(m.dst), ring_start=i32(m.ring_start),
        replay_prefix_len=i32(m.prefix), active_request_indices=i32(m.active if active is None else active),
        rand_seed=torch.tensor([seed if seed is not None else 0], dtype=torch.int64, device=device)
        if dp.spec.philox_rounds > 0 else None)


def materialize(dp: ri.DeviceProblem, tabs: Tables, max_workgroups: int = 0, stream=None,
                active=None) -> None:
    """One library call on a device problem (enqueue only)."""
    from replayssm_persistent_rssm_amd import rssm_materialize
    s = dp.spec
    rssm_materialize(
        tabs.state_ptrs, tabs.state_slot_strides, tabs.x_cache_ptrs, tabs.x_cache_slot_strides,
        tabs.B_cache_ptrs, tabs.B_cache_slot_strides, tabs.dt_cache_ptrs, tabs.dt_cache_slot_strides,
        tabs.A_ptrs, tabs.state_scale_ptrs, tabs.state_scale_slot_strides, tabs.src_slots, tabs.dst_slots,
        tabs.ring_start, tabs.replay_prefix_len,
        tabs.active_request_indices if active is None else active,
        state_dtype=s.state_dtype, input_dtype=s.input_dtype, matrixA_dtype="f32", dim=s.dim, dstate=s.dstate,
        num_heads=s.H, heads_per_group=s.hpg, max_window=s.W, ring_buffer_len=s.R, pad_slot_id=s.pad_slot_id,
        rand_seed=tabs.rand_seed, philox_rounds=s.philox_rounds, max_workgroups=max_workgroups, stream=stream)


def prepared(dp: ri.DeviceProblem, tabs: Tables, max_workgroups: int = 0, stream=None,
             replay_prefix_len=None):
    """A MaterializeCall for a device problem: marshalled once, one C call per
    invocation (optionally with another prefix-length tensor)."""
    from replayssm_persistent_rssm_amd import MaterializeCall
    s = dp.spec
    return MaterializeCall(
        tabs.state_ptrs, tabs.state_slot_strides, tabs.x_cache_ptrs, tabs.x_cache_slot_strides,
        tabs.B_cache_ptrs, tabs.B_cache_slot_strides, tabs.dt_cache_ptrs, tabs.dt_cache_slot_strides,
        tabs.A_ptrs, tabs.state_scale_ptrs, tabs.state_scale_slot_strides, tabs.src_slots, tabs.dst_slots,
        tabs.ring_start, tabs.replay_prefix_len if replay_prefix_len is None else replay_prefix_len,
        tabs.active_request_indices,
        state_dtype=s.state_dtype, input_dtype=s.input_dtype, matrixA_dtype="f32", dim=s.dim, dstate=s.dstate,
        num_heads=s.H, heads_per_group=s.hpg, max_window=s.W, ring_buffer_len=s.R, pad_slot_id=s.pad_slot_id,
        rand_seed=tabs.rand_seed, philox_rounds=s.philox_rounds, max_workgroups=max_workgroups, stream=stream)


def algorithmic_bytes(spec: ri.Spec, meta: ri.Meta, n_active: Optional[int] = None) -> int:
    """Bytes the method itself must move for one call: per written (layer,
    request) the state in and out (+ row scales for one-byte state) and, for
    k > 0, the k replayed x, B and dt rows; plus A per layer touched."""
    sb = ri.ELEM_BYTES[spec.state_dtype]
    ib = ri.ELEM_BYTES[spec.input_dtype]
    total = 0
    layers = set()
    n = int((meta.active >= 0).cumprod().sum()) if n_active is None else n_active
    for i in range(n):
        b = int(meta.active[i])
        k = int(meta.prefix[b])
        for l in range(spec.L):
            s, d = meta.src[l, b], meta.dst[l, b]
            if s == spec.pad_slot_id or d == spec.pad_slot_id:
                continue
            layers.add(l)
            total += 2 * spec.H * spec.dim * spec.dstate * sb
            if ri.one_byte(spec.state_dtype):
                total += 2 * spec.H * spec.dim * 4
            total += k * (spec.H * spec.dim * ib + spec.G * spec.dstate * ib + spec.H * 4)
    return total + len(layers) * spec.H * 4


def prepared_checkpoints(dp: ri.DeviceProblem, tabs: Tables, dst, prefix, max_workgroups: int = 0, stream=None):
    """A multi-checkpoint MaterializeCall: dst (C, L, B) and prefix (C, B)
    device int32 tensors replace the problem's destination and prefix tables."""
    from replayssm_persistent_rssm_amd import MaterializeCall
    s = dp.spec
    return MaterializeCall(
        tabs.state_ptrs, tabs.state_slot_strides, tabs.x_cache_ptrs, tabs.x_cache_slot_strides,
        tabs.B_cache_ptrs, tabs.B_cache_slot_strides, tabs.dt_cache_ptrs, tabs.dt_cache_slot_strides,
        tabs.A_ptrs, tabs.state_scale_ptrs, tabs.state_scale_slot_strides, tabs.src_slots, dst,
        tabs.ring_start, prefix, tabs.active_request_indices,
        state_dtype=s.state_dtype, input_dtype=s.input_dtype, matrixA_dtype="f32", dim=s.dim, dstate=s.dstate,
        num_heads=s.H, heads_per_group=s.hpg, max_window=s.W, ring_buffer_len=s.R, pad_slot_id=s.pad_slot_id,
        rand_seed=tabs.rand_seed, philox_rounds=s.philox_rounds, max_workgroups=max_workgroups, stream=stream,
        checkpoints=True)


def checkpoint_bytes(spec: ri.Spec, meta: ri.Meta, dst: np.ndarray, prefix: np.ndarray) -> int:
    """Bytes a multi-checkpoint call must move: per (layer, request) with a
    live source and at least one live destination, the source state once (+
    row scales), every live checkpoint's state written (+ scales), and the
    replayed x, B and dt rows of the longest live prefix; plus A per layer."""
    sb = ri.ELEM_BYTES[spec.state_dtype]
    ib = ri.ELEM_BYTES[spec.input_dtype]
    tile = spec.H * spec.dim * spec.dstate * sb + (spec.H * spec.dim * 4 if ri.one_byte(spec.state_dtype) else 0)
    total = 0
    layers = set()
    n = int((meta.active >= 0).cumprod().sum())
    for i in range(n):
        b = int(meta.active[i])
        for l in range(spec.L):
            if meta.src[l, b] == spec.pad_slot_id:
                continue
            live = [c for c in range(dst.shape[0]) if dst[c, l, b] != spec.pad_slot_id]
            if not live:
                continue
            layers.add(l)
            k = max(int(prefix[c, b]) for c in live)
            total += tile * (1 + len(live))
            total += k * (spec.H * spec.dim * ib + spec.G * spec.dstate * ib + spec.H * 4)
    return total + len(layers) * spec.H * 4


def flush_and_checkpoint_tables(meta: ri.Meta):
    """Two checkpoints per request: 0 applies every buffered token in place
    (destination = source slot, the request's prefix length); 1 writes the
    state at half that prefix to the request's destination slot."""
    dst = np.stack([meta.src, meta.dst]).astype(np.int32)
    pre = np.stack([meta.prefix, meta.prefix // 2]).astype(np.int32)
    return dst, pre


def gdn_bytes(spec: ri.GdnSpec, idx, acc, tidx=None, tstep=None) -> int:
    """Bytes a gated-delta-rule commit must move: per committed (request,
    layer, value head) the fp32 state read and written (+ written once more for
    a tracked step inside the prefix) and the n accepted tokens' value rows, g
    and beta; per (request, layer, key head) the n key rows."""
    tile = spec.dv * spec.dk * 4
    total = 0
    for b in range(spec.B):
        n = int(acc[b])
        if int(idx[b]) <= spec.null_block_id or n <= 0:
            continue
        n = min(n, spec.T)
        tracked = tidx is not None and int(tidx[b]) > spec.null_block_id and 0 <= int(tstep[b]) < n
        per_head = 2 * tile + (tile if tracked else 0) + n * (spec.dv * 2 + 8)
        total += spec.L * (spec.HV * per_head + spec.H * n * spec.dk * 2)
    return total


# --------------------------------------------------------------------------
# Decode step
# --------------------------------------------------------------------------
def _ssu_args(d: ri.SsuDeviceProblem, max_workgroups: int = 0):
    spec = d.spec
    args = (d.state, d.x_ring, d.B_ring, d.dt_ring, d.A, d.x_new, d.B_new, d.C_new, d.dt_new, d.y, d.slots,
            d.ring_start, d.num_buffered)
    kw = dict(ring_buffer_len=spec.R, D=d.D, dt_bias=d.dt_bias, z=d.z, dt_softplus=spec.dt_softplus,
              pad_slot_id=spec.pad_slot_id, max_workgroups=max_workgroups)
    return args, kw


def ssu_call(d: ri.SsuDeviceProblem, max_workgroups: int = 0, stream=None) -> None:
    """One rssm_ssu_decode call on a device problem (enqueued, not synchronised)."""
    import replayssm_persistent_rssm_amd as rp
    args, kw = _ssu_args(d, max_workgroups)
    rp.rssm_ssu_decode(*args, stream=stream, **kw)


def ssu_prepared(d: ri.SsuDeviceProblem, max_workgroups: int = 0, stream=None):
    """The same call, marshalled once (a callable that makes one C call)."""
    import replayssm_persistent_rssm_amd as rp
    args, kw = _ssu_args(d, max_workgroups)
    return rp.SsuDecodeCall(*args, stream=stream, **kw)


def _host_storage(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def ssu_download(d: ri.SsuDeviceProblem):
    """(x_ring, B_ring, dt_ring, y) in host storage form after a call."""
    it = d.spec.input_dtype
    return (_host_storage(d.x_ring, it), _host_storage(d.B_ring, it), d.dt_ring.cpu().numpy(), d.y.cpu().numpy())


def ssu_bytes(spec: ri.SsuSpec, slots, num_buffered) -> int:
    """Bytes a decode step must move: per live request the checkpoint tiles
    (read), the n pending ring entries (x, dt per head; B per group; read),
    the T new tokens' inputs (x, z, dt per head; B, C per group; read), the
    outputs (fp32, written) and the ring append (x, dt per head; B per group;
    written); plus A, D and dt_bias once."""
    sb = {"f32": 4, "bf16": 2, "f16": 2}[spec.state_dtype]
    ib = {"f32": 4, "bf16": 2, "f16": 2}[spec.input_dtype]
    H, G, T, dim, ds = spec.H, spec.G, spec.T, spec.dim, spec.dstate
    x_row, b_row = dim * ib, ds * ib
    total = 3 * H * 4
    for b in range(spec.B):
        if int(slots[b]) == spec.pad_slot_id:
            continue
        n = int(num_buffered[b])
        total += H * dim * ds * sb                                       # checkpoint
        total += n * (H * (x_row + 4) + G * b_row)                       # pending entries
        total += T * (H * (x_row * (2 if spec.has_z else 1) + 4) + 2 * G * b_row)   # new inputs
        total += T * H * dim * 4                                         # outputs
        total += T * (H * (x_row + 4) + G * b_row)                       # ring append
    return total

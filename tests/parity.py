"""Element-by-element comparison of the HIP path against the CPU oracle.

Tolerances (written here, per the method's arithmetic):
  * bytes that the call must not write (other slots, stride gaps, sources,
    rings), zero-prefix copies, skips: bit-exact;
  * fp32 state: |gpu - exact| <= 1e-5 * M, where M = D|S0| + sum_j w_j |x_j B_j|
    is the oracle's per-element magnitude sum (|exact| when nothing cancels);
  * bf16 / fp16 state: the GPU code is the oracle's code or its neighbour in
    value order (one unit in the last place), or -- where cancellation makes
    one ulp finer than fp32 accumulation can resolve -- within
    1e-5 * M + half an ulp of the exact value;
  * int8 / e4m3 state: codes within one step in value order of the oracle's,
    row scales within 1e-5 relative of the oracle's;
  * NaN: the GPU's code is a NaN code of the format exactly where the
    oracle's is, of either sign (and any payload).  IEEE 754 leaves the sign
    and payload of a NaN that arithmetic produces unspecified, so only the
    NaN-ness is unique.  int8 encodes NaN as 0, which is compared as a code;
  * an infinite exact value (an infinity in the inputs) in fp32 / bf16 / fp16
    state: the GPU's value is that same infinity (M is infinite there, so the
    relative bound would accept anything).
The fp32 accumulation error of the GPU fold is bounded by a few ulps of fp32
times M (k <= 16 fused multiply-adds plus one exp per token), far inside
1e-5 * M.
"""
from __future__ import annotations

import numpy as np

import oracle
import rssm_inputs as ri


def ordered_index(dtype: str, codes: np.ndarray) -> np.ndarray:
    """Position of each code in value order (sign-magnitude; +0 and -0 -> 0)."""
    c = np.asarray(codes)
    if dtype == "i8":
        return c.view(np.int8).astype(np.int64)
    if dtype == "f8e4m3":
        u = c.view(np.uint8).astype(np.int64)
        mag, neg = u & 0x7F, (u & 0x80) != 0
    else:
        u = c.view(np.uint16).astype(np.int64)
        mag, neg = u & 0x7FFF, (u & 0x8000) != 0
    return np.where(neg, -mag, mag)


def ulp_at(dtype: str, v: np.ndarray) -> np.ndarray:
    mant, emin = {"bf16": (7, -126), "f16": (10, -14)}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(v), 1e-300)))
    return 2.0 ** (np.maximum(e, emin) - mant)


def nan_codes(dtype: str, codes: np.ndarray) -> np.ndarray:
    """Per element: is the code a NaN of the format (any sign, any payload)?"""
    c = np.asarray(codes)
    if dtype == "i8":
        return np.zeros(c.view(np.int8).shape, bool)
    if dtype == "f8e4m3":
        return (c.view(np.uint8) & 0x7F) == 0x7F
    if dtype == "f32":
        return np.isnan(c.view(np.float32))
    exp_mask, mant_mask = {"bf16": (0x7F80, 0x007F), "f16": (0x7C00, 0x03FF)}[dtype]
    u = c.view(np.uint16)
    return ((u & exp_mask) == exp_mask) & ((u & mant_mask) != 0)


def compare_tile(dtype: str, got, exp_codes, exact, mag, got_scale=None, exp_scale=None, what=""):
    """Compare one written region (k > 0) of codes (and row scales)."""
    got = np.asarray(got).reshape(-1)
    exp_codes = np.asarray(exp_codes).reshape(-1)
    en, gn = nan_codes(dtype, exp_codes), nan_codes(dtype, got)
    assert np.array_equal(gn, en), (f"{what}: NaN elements differ ({(en & ~gn).sum()} NaN in the oracle only, "
                                    f"{(gn & ~en).sum()} on the GPU only)")
    if en.any():
        # the rest as usual; the NaN elements compare equal from here on
        exact = np.where(en.reshape(np.shape(exact)), 0.0, exact)
        mag = np.where(en.reshape(np.shape(mag)), 0.0, mag)
        got, exp_codes = _zero_elements(dtype, got, en), _zero_elements(dtype, exp_codes, en)
    exact = np.asarray(exact, np.float64).reshape(-1)
    mag = np.asarray(mag, np.float64).reshape(-1)
    if dtype == "f32":
        g = got.view(np.float32).astype(np.float64)
        with np.errstate(invalid="ignore"):   # inf - inf where both hold the same infinity
            err = np.abs(g - exact)
        bad = ~((err <= 1e-5 * mag) | (g == exact)) | (np.isinf(exact) & (g != exact))
        if bad.any():
            with np.errstate(invalid="ignore"):
                worst = (err / np.maximum(mag, 1e-300))[bad].max()
            raise AssertionError(f"{what}: {bad.sum()} fp32 elements beyond 1e-5*M; worst {worst:.3e}")
        return
    di = np.abs(ordered_index(dtype, got) - ordered_index(dtype, exp_codes))
    if dtype in ("bf16", "f16"):
        g = oracle.decode(dtype, got.view(np.uint16)) if got.size <= 4096 else _fast_decode(dtype, got)
        with np.errstate(invalid="ignore"):   # inf - inf: not near, decided by the code step
            near = np.abs(g - exact) <= 1e-5 * mag + 0.5 * ulp_at(dtype, np.maximum(np.abs(g), np.abs(exact)))
        bad = ~((di <= 1) | near) | (np.isinf(exact) & (g != exact))
        assert not bad.any(), f"{what}: {bad.sum()} {dtype} codes off by more than 1 ulp (max {di.max()})"
        return
    bad = di > 1
    assert not bad.any(), f"{what}: {bad.sum()} {dtype} codes more than one step off (max {di.max()})"
    if got_scale is not None:
        gs = np.asarray(got_scale, np.float64).reshape(-1)
        es = np.asarray(exp_scale, np.float64).reshape(-1)
        rel = np.abs(gs - es) / np.maximum(np.abs(es), 1e-300)
        assert np.all(rel <= 1e-5), f"{what}: row scales differ by up to {rel.max():.3e}"


def _zero_elements(dtype: str, codes: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """A copy of the codes with the masked elements set to the code of +0."""
    view = {"f8e4m3": np.uint8, "bf16": np.uint16, "f16": np.uint16, "f32": np.uint32}[dtype]
    out = np.array(codes, copy=True)
    out.view(view)[mask] = 0
    return out


def _fast_decode(dtype: str, codes: np.ndarray) -> np.ndarray:
    """Library cast (torch) for large arrays; the oracle's decoder is pinned to it."""
    import torch
    c = np.ascontiguousarray(codes).view(np.int16)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return torch.from_numpy(c).view(tdt).to(torch.float64).numpy()


def written_pairs(prob):
    m, s = prob.meta, prob.spec
    out = []
    for i in range(s.B):
        b = int(m.active[i])
        if b < 0 or b >= s.B:
            break
        for l in range(s.L):
            src, dst = int(m.src[l, b]), int(m.dst[l, b])
            if src == s.pad_slot_id or dst == s.pad_slot_id:
                continue
            out.append((l, b, src, dst))
    return out


def check_against_oracle(prob, gpu_state, gpu_scale, expected=None):
    """Full comparison of the GPU's state/scale pools with the oracle's."""
    spec = prob.spec
    st_o, sc_o, ex, mg = expected if expected is not None else oracle.materialize(prob, want_exact=True)
    n = spec.H * spec.dim * spec.dstate
    ns = spec.H * spec.dim
    written = [np.zeros(a.shape[0], bool) for a in prob.state]
    for l, b, s, d in written_pairs(prob):
        written[l][d] = True
        k = int(prob.meta.prefix[b])
        what = f"layer {l} request {b} slot {s}->{d} k={k}"
        if k == 0:
            assert np.array_equal(gpu_state[l][d, :n].view(np.uint8), prob.state[l][s, :n].view(np.uint8)), what
            if gpu_scale is not None:
                assert np.array_equal(gpu_scale[l][d, :ns].view(np.uint32), prob.scale[l][s, :ns].view(np.uint32)), what
        else:
            compare_tile(spec.state_dtype, gpu_state[l][d, :n], st_o[l][d, :n], ex[l][d, :n], mg[l][d, :n],
                         gpu_scale[l][d, :ns] if gpu_scale is not None else None,
                         sc_o[l][d, :ns] if sc_o is not None else None, what)
        # the gap after the dense tile in the destination slot is untouched
        assert np.array_equal(gpu_state[l][d, n:].view(np.uint8), prob.state[l][d, n:].view(np.uint8)), what
        if gpu_scale is not None:
            assert np.array_equal(gpu_scale[l][d, ns:].view(np.uint8), prob.scale[l][d, ns:].view(np.uint8)), what
    for l in range(spec.L):
        keep = ~written[l]
        assert np.array_equal(gpu_state[l][keep].view(np.uint8), prob.state[l][keep].view(np.uint8)), \
            f"layer {l}: a slot that is not a destination changed"
        if gpu_scale is not None:
            assert np.array_equal(gpu_scale[l][keep].view(np.uint8), prob.scale[l][keep].view(np.uint8)), \
                f"layer {l}: a scale slot that is not a destination changed"
    return st_o, sc_o, ex, mg


def checkpoint_writes(prob, dst, pre):
    """(c, l, b, src, dst_slot, k) of every checkpoint write of a call."""
    m, s = prob.meta, prob.spec
    out = []
    for i in range(s.B):
        b = int(m.active[i])
        if b < 0 or b >= s.B:
            break
        for l in range(s.L):
            src = int(m.src[l, b])
            if src == s.pad_slot_id:
                continue
            for c in range(dst.shape[0]):
                d = int(dst[c, l, b])
                if d != s.pad_slot_id:
                    out.append((c, l, b, src, d, int(pre[c, b])))
    return out


def check_checkpoints_against_oracle(prob, dst, pre, gpu_state, gpu_scale, expected=None):
    """Full comparison of a multi-checkpoint call's pools with the oracle's."""
    spec = prob.spec
    st_o, sc_o, ex, mg = expected if expected is not None else oracle.materialize_checkpoints(
        prob, list(dst), list(pre), want_exact=True)
    n = spec.H * spec.dim * spec.dstate
    ns = spec.H * spec.dim
    written = [np.zeros(a.shape[0], bool) for a in prob.state]
    for c, l, b, s, d, k in checkpoint_writes(prob, dst, pre):
        written[l][d] = True
        what = f"checkpoint {c} layer {l} request {b} slot {s}->{d} k={k}"
        if k == 0:
            assert np.array_equal(gpu_state[l][d, :n].view(np.uint8), prob.state[l][s, :n].view(np.uint8)), what
            if gpu_scale is not None:
                assert np.array_equal(gpu_scale[l][d, :ns].view(np.uint32), prob.scale[l][s, :ns].view(np.uint32)), what
        else:
            compare_tile(spec.state_dtype, gpu_state[l][d, :n], st_o[l][d, :n], ex[l][d, :n], mg[l][d, :n],
                         gpu_scale[l][d, :ns] if gpu_scale is not None else None,
                         sc_o[l][d, :ns] if sc_o is not None else None, what)
        assert np.array_equal(gpu_state[l][d, n:].view(np.uint8), prob.state[l][d, n:].view(np.uint8)), what
        if gpu_scale is not None:
            assert np.array_equal(gpu_scale[l][d, ns:].view(np.uint8), prob.scale[l][d, ns:].view(np.uint8)), what
    for l in range(spec.L):
        keep = ~written[l]
        assert np.array_equal(gpu_state[l][keep].view(np.uint8), prob.state[l][keep].view(np.uint8)), \
            f"layer {l}: a slot that is not a destination changed"
        if gpu_scale is not None:
            assert np.array_equal(gpu_scale[l][keep].view(np.uint8), prob.scale[l][keep].view(np.uint8)), \
                f"layer {l}: a scale slot that is not a destination changed"
    return st_o, sc_o, ex, mg

"""The oracle's materialize pinned to what the pages and the mathematics fix.

The pages (flashinfer.mamba.replayssm_materialize, Parameters and Notes) fix:
a zero prefix is an exact state/scale copy; a (layer, request) with a pad slot
in either table is skipped; requests after the first -1 of the active list are
not touched; the source state and ring are read-only; ring entries start at
ring_start and wrap modulo ring_buffer_len.  The recurrence
S <- exp(dt*A) S + dt x B^T fixes closed forms: A = 0 and S0 = 0 gives the
matrix product X^T diag(dt) B; x = 0 gives pure decay exp(A sum dt) S0;
constant inputs give a geometric series; in general the result is the
unrolled sum D S0 + sum_j w_j x_j B_j^T with D = prod a_j and
w_j = dt_j prod_{u>j} a_u.  Applying k1 then k2 tokens equals applying k1+k2.
"""
import hashlib

import numpy as np
import pytest

import rssm_inputs as ri

SMALL = ri.Spec("pin_small", L=2, B=4, H=4, hpg=2, dim=8, dstate=16, R=8, W=8,
                state_dtype="f32", input_dtype="f32", k_lo=0, k_hi=8, slots=8, ring_slots=8,
                slot_mode="perm", stride_pad="per_layer")


def tile_view(pool, stride, slot, h, spec):
    n = spec.dim * spec.dstate
    return pool[slot, h * n:(h + 1) * n].reshape(spec.dim, spec.dstate)


def ring_views(prob, l, slot):
    """Dense per-slot ring views (x [R,H,dim], B [R,G,dstate], dt [R,H]) as fp64."""
    import oracle
    s = prob.spec
    _, _, d_x, d_B, d_dt = ri.dense_sizes(s)
    x = oracle.decode(s.input_dtype, prob.x[l][slot, :d_x]).reshape(s.R, s.H, s.dim)
    B = oracle.decode(s.input_dtype, prob.Bm[l][slot, :d_B]).reshape(s.R, s.G, s.dstate)
    dt = prob.dt[l][slot, :d_dt].astype(np.float64).reshape(s.R, s.H)
    return x, B, dt


def written_pairs(prob):
    m = prob.meta
    out = []
    for i in range(prob.spec.B):
        b = int(m.active[i])
        if b == -1:
            break
        for l in range(prob.spec.L):
            s, d = int(m.src[l, b]), int(m.dst[l, b])
            if s == prob.spec.pad_slot_id or d == prob.spec.pad_slot_id:
                continue
            out.append((l, b, s, d))
    return out


def sha(arrs):
    h = hashlib.sha256()
    for a in arrs:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_zero_prefix_is_exact_copy(orc):
    spec = ri.with_(SMALL, state_dtype="bf16", prefix=[0, 0, 3, 0])
    prob = ri.make_problem(spec, 21)
    st, _, _, _ = orc.materialize(prob)
    n = spec.H * spec.dim * spec.dstate
    for l, b, s, d in written_pairs(prob):
        if prob.meta.prefix[b] == 0:
            assert np.array_equal(st[l][d, :n].view(np.uint16), prob.state[l][s, :n].view(np.uint16))


@pytest.mark.parametrize("dtype", ["i8", "f8e4m3"])
def test_zero_prefix_copies_codes_and_scales(orc, dtype):
    spec = ri.with_(SMALL, state_dtype=dtype, input_dtype="bf16", prefix=[0, 2, 0, 0])
    prob = ri.make_problem(spec, 22)
    st, sc, _, _ = orc.materialize(prob)
    n, ns = spec.H * spec.dim * spec.dstate, spec.H * spec.dim
    for l, b, s, d in written_pairs(prob):
        if prob.meta.prefix[b] == 0:
            assert np.array_equal(st[l][d, :n], prob.state[l][s, :n])
            assert np.array_equal(sc[l][d, :ns].view(np.uint32), prob.scale[l][s, :ns].view(np.uint32))


def _written_mask(prob):
    """Per layer: boolean mask of state-pool elements the call may write."""
    s = prob.spec
    n = s.H * s.dim * s.dstate
    masks = [np.zeros(a.shape, bool) for a in prob.state]
    smasks = [np.zeros(a.shape, bool) for a in prob.scale] if prob.scale else None
    for l, b, src, dst in written_pairs(prob):
        masks[l][dst, :n] = True
        if smasks:
            smasks[l][dst, :s.H * s.dim] = True
    return masks, smasks


@pytest.mark.parametrize("dtype", ["f32", "i8"])
def test_pad_and_inactive_untouched(orc, dtype):
    spec = ri.with_(SMALL, state_dtype=dtype, B=6, slots=16, ring_slots=16, n_active=4, pad_frac=0.25)
    prob = ri.make_problem(spec, 23)
    st, sc, _, _ = orc.materialize(prob)
    masks, smasks = _written_mask(prob)
    assert any(m.any() for m in masks)
    for l in range(spec.L):
        assert np.array_equal(st[l][~masks[l]], prob.state[l][~masks[l]])   # includes stride gaps
        if sc:
            assert np.array_equal(sc[l][~smasks[l]], prob.scale[l][~smasks[l]])
    # every (layer, request) that is listed and unpadded did change
    n = spec.H * spec.dim * spec.dstate
    for l, b, s, d in written_pairs(prob):
        if prob.meta.prefix[b] > 0:
            assert not np.array_equal(st[l][d, :n], prob.state[l][d, :n])


def test_requests_after_first_minus_one_are_ignored(orc):
    spec = ri.with_(SMALL, B=4, n_active=4)
    prob = ri.make_problem(spec, 24)
    prob.meta.active[2] = -1           # entries after the first -1 must not count
    st, _, _, _ = orc.materialize(prob)
    n = spec.H * spec.dim * spec.dstate
    for b in prob.meta.active[3:4]:
        for l in range(spec.L):
            d = prob.meta.dst[l, b]
            assert np.array_equal(st[l][d, :n], prob.state[l][d, :n])


def test_nondefault_pad_makes_slot_zero_valid(orc):
    spec = ri.with_(SMALL, slot_mode="fixed", B=2, src_fixed=[0, 7], dst_fixed=[3, 4], pad_slot_id=7,
                    prefix=[2, 2], active_order="sorted", stride_pad="none")
    prob = ri.make_problem(spec, 25)
    st, _, _, _ = orc.materialize(prob)
    n = spec.H * spec.dim * spec.dstate
    for l in range(spec.L):
        assert not np.array_equal(st[l][3, :n], prob.state[l][3, :n])   # src slot 0 used
        assert np.array_equal(st[l][4, :n], prob.state[l][4, :n])       # src == pad 7: skipped


def test_inputs_read_only(orc):
    spec = ri.with_(SMALL, state_dtype="f8e4m3", input_dtype="bf16", philox_rounds=10, rand_seed=5)
    prob = ri.make_problem(spec, 26)
    before = sha(prob.state + prob.scale + prob.x + prob.Bm + prob.dt + prob.A +
                 [prob.meta.src, prob.meta.dst, prob.meta.ring_start, prob.meta.prefix, prob.meta.active])
    orc.materialize(prob)
    after = sha(prob.state + prob.scale + prob.x + prob.Bm + prob.dt + prob.A +
                [prob.meta.src, prob.meta.dst, prob.meta.ring_start, prob.meta.prefix, prob.meta.active])
    assert before == after


def test_ring_wrap_equals_unrolled_ring(orc):
    """tiny_f32 request 1 starts at entry 6 of an 8-entry ring and applies 5:
    entries 6,7,0,1,2.  Rotating that slot's ring so the same entries sit at
    0..4 and starting at 0 must give the identical bytes."""
    spec = ri.CONFIGS["tiny_f32"]
    prob = ri.make_problem(spec, 1000)
    st, _, ex, _ = orc.materialize(prob, want_exact=True)
    prob2 = ri.make_problem(spec, 1000)
    _, _, d_x, d_B, d_dt = ri.dense_sizes(spec)
    s = int(prob.meta.src[0, 1])
    r0 = int(prob.meta.ring_start[1])
    assert (r0, int(prob.meta.prefix[1])) == (6, 5)
    for arr, d, w in ((prob2.x[0], d_x, spec.H * spec.dim), (prob2.Bm[0], d_B, spec.G * spec.dstate),
                      (prob2.dt[0], d_dt, spec.H)):
        ring = arr[s, :d].reshape(spec.R, w)
        arr[s, :d] = np.roll(ring, -r0, axis=0).reshape(-1)
    prob2.meta.ring_start[1] = 0
    st2, _, ex2, _ = orc.materialize(prob2, want_exact=True)
    dslot = int(prob.meta.dst[0, 1])
    assert np.array_equal(st[0][dslot], st2[0][dslot])
    assert np.array_equal(ex[0][dslot], ex2[0][dslot])


def decode_independent(dtype, codes):
    """Stored codes as fp64 values without the oracle: numpy for fp32/int8,
    torch's CPU casts for bf16, fp16 and OCP e4m3fn."""
    import torch
    codes = np.ascontiguousarray(codes)
    if dtype == "f32":
        return codes.view(np.float32).astype(np.float64)
    if dtype == "i8":
        return codes.view(np.int8).astype(np.float64)
    tdt = {"bf16": (torch.int16, torch.bfloat16), "f16": (torch.int16, torch.float16),
           "f8e4m3": (torch.uint8, torch.float8_e4m3fn)}[dtype]
    raw = torch.from_numpy(codes.view(np.int16 if tdt[0] == torch.int16 else np.uint8).copy())
    return raw.view(tdt[1]).to(torch.float64).numpy()


def spread_row_scales(prob, seed):
    """Replace every row scale of every slot (sources, destinations, gaps) by
    an independent power of two in [2^-8, 2^8] times U[1, 2): a scale read
    from the wrong row, the wrong slot, or not applied at all changes the
    dequantized state by a large factor."""
    rng = np.random.default_rng(seed)
    for sc in prob.scale:
        sc[:] = (np.exp2(rng.integers(-8, 9, size=sc.shape)) * rng.uniform(1.0, 2.0, size=sc.shape)).astype(np.float32)


def _unrolled(prob, l, b, s, h):
    """D*S0 + sum_j w_j x_j B_j^T in fp64 (closed form of the recurrence).
    One-byte sources dequantize as code times the source slot's row scale
    (the materialize page's state_scale_ptrs hold the quantized state's
    scales; the pull-request page's change table reads them as the decode
    scale input), decoded here without the oracle."""
    spec = prob.spec
    k, r0 = int(prob.meta.prefix[b]), int(prob.meta.ring_start[b])
    x, B, dt = ring_views(prob, l, s)
    n = spec.dim * spec.dstate
    S0 = decode_independent(spec.state_dtype, prob.state[l][s, h * n:(h + 1) * n]).reshape(spec.dim, spec.dstate)
    if prob.scale:
        S0 = S0 * prob.scale[l][s, h * spec.dim:(h + 1) * spec.dim].astype(np.float64)[:, None]
    A = float(prob.A[l][h])
    g = h // spec.hpg
    es = [(r0 + j) % spec.R for j in range(k)]
    a = np.array([np.exp(dt[e, h] * A) for e in es])
    D = np.prod(a)
    out = D * S0
    for j, e in enumerate(es):
        w = dt[e, h] * np.prod(a[j + 1:])
        out = out + w * np.outer(x[e, h], B[e, g])
    return out


@pytest.mark.parametrize("dtype", ["f32", "i8", "f8e4m3"])
@pytest.mark.parametrize("k", [1, 3, 8])
def test_unrolled_sum_and_single_step(orc, k, dtype):
    spec = ri.with_(SMALL, prefix=[k] * 4, state_dtype=dtype, input_dtype="f32" if dtype == "f32" else "bf16")
    prob = ri.make_problem(spec, 27 + k)
    if prob.scale:
        spread_row_scales(prob, 270 + k)
    _, _, ex, _ = orc.materialize(prob, want_exact=True)
    n = spec.dim * spec.dstate
    for l, b, s, d in written_pairs(prob):
        for h in range(spec.H):
            ref = _unrolled(prob, l, b, s, h)
            got = ex[l][d, h * n:(h + 1) * n].reshape(spec.dim, spec.dstate)
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_closed_form_gemm_when_A_and_S0_zero(orc):
    spec = ri.with_(SMALL, prefix=[5, 8, 1, 3])
    prob = ri.make_problem(spec, 31)
    for l in range(spec.L):
        prob.A[l][:] = 0.0
        prob.state[l][:] = 0.0
    _, _, ex, _ = orc.materialize(prob, want_exact=True)
    n = spec.dim * spec.dstate
    for l, b, s, d in written_pairs(prob):
        x, B, dt = ring_views(prob, l, s)
        k, r0 = int(prob.meta.prefix[b]), int(prob.meta.ring_start[b])
        es = [(r0 + j) % spec.R for j in range(k)]
        for h in range(spec.H):
            X = np.stack([x[e, h] for e in es])                   # k x dim
            Bk = np.stack([B[e, h // spec.hpg] for e in es])      # k x dstate
            ref = X.T @ np.diag([dt[e, h] for e in es]) @ Bk
            got = ex[l][d, h * n:(h + 1) * n].reshape(spec.dim, spec.dstate)
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_closed_form_pure_decay_when_x_zero(orc):
    spec = ri.with_(SMALL, prefix=[4, 7, 2, 8])
    prob = ri.make_problem(spec, 32)
    for l in range(spec.L):
        prob.x[l][:] = 0.0
    _, _, ex, _ = orc.materialize(prob, want_exact=True)
    n = spec.dim * spec.dstate
    for l, b, s, d in written_pairs(prob):
        _, _, dt = ring_views(prob, l, s)
        k, r0 = int(prob.meta.prefix[b]), int(prob.meta.ring_start[b])
        for h in range(spec.H):
            tot = sum(dt[(r0 + j) % spec.R, h] for j in range(k))
            ref = np.exp(float(prob.A[l][h]) * tot) * prob.state[l][s, h * n:(h + 1) * n].astype(np.float64)
            np.testing.assert_allclose(ex[l][d, h * n:(h + 1) * n], ref, rtol=1e-12)


@pytest.mark.parametrize("dtype", ["i8", "f8e4m3"])
def test_one_byte_source_pure_decay(orc, dtype):
    """x = 0 on a one-byte source: every element of the result is
    exp(A_h * sum_j dt_j) * code[r, c] * scale_src[r], with codes decoded by
    numpy / torch and row scales spread over 2^-8 .. 2^9.  A scale taken by
    column, from the destination slot, or left out fails here."""
    spec = ri.with_(SMALL, state_dtype=dtype, input_dtype="bf16", prefix=[4, 7, 2, 8])
    prob = ri.make_problem(spec, 35)
    spread_row_scales(prob, 350)
    for l in range(spec.L):
        prob.x[l][:] = 0
    _, _, ex, _ = orc.materialize(prob, want_exact=True)
    n = spec.dim * spec.dstate
    checked = 0
    for l, b, s, d in written_pairs(prob):
        _, _, dt = ring_views(prob, l, s)
        k, r0 = int(prob.meta.prefix[b]), int(prob.meta.ring_start[b])
        assert k > 0
        for h in range(spec.H):
            tot = sum(dt[(r0 + j) % spec.R, h] for j in range(k))
            codes = decode_independent(dtype, prob.state[l][s, h * n:(h + 1) * n]).reshape(spec.dim, spec.dstate)
            rows = prob.scale[l][s, h * spec.dim:(h + 1) * spec.dim].astype(np.float64)
            ref = np.exp(float(prob.A[l][h]) * tot) * codes * rows[:, None]
            np.testing.assert_allclose(ex[l][d, h * n:(h + 1) * n].reshape(spec.dim, spec.dstate), ref, rtol=1e-12)
            checked += 1
    assert checked > 0


def test_closed_form_geometric_series(orc):
    spec = ri.with_(SMALL, prefix=[8, 6, 3, 1])
    prob = ri.make_problem(spec, 33)
    for l in range(spec.L):
        xr = prob.x[l].copy()
        # constant ring: every entry of every slot equals entry 0
        _, _, d_x, d_B, d_dt = ri.dense_sizes(spec)
        for arr, d, w in ((prob.x[l], d_x, spec.H * spec.dim), (prob.Bm[l], d_B, spec.G * spec.dstate),
                          (prob.dt[l], d_dt, spec.H)):
            ring = arr[:, :d].reshape(arr.shape[0], spec.R, w)
            arr[:, :d] = np.repeat(ring[:, :1], spec.R, axis=1).reshape(arr.shape[0], d)
        del xr
    _, _, ex, _ = orc.materialize(prob, want_exact=True)
    n = spec.dim * spec.dstate
    for l, b, s, d in written_pairs(prob):
        x, B, dt = ring_views(prob, l, s)
        k = int(prob.meta.prefix[b])
        for h in range(spec.H):
            a = np.exp(dt[0, h] * float(prob.A[l][h]))
            S0 = prob.state[l][s, h * n:(h + 1) * n].astype(np.float64).reshape(spec.dim, spec.dstate)
            ref = a**k * S0 + dt[0, h] * (1 - a**k) / (1 - a) * np.outer(x[0, h], B[0, h // spec.hpg])
            np.testing.assert_allclose(ex[l][d, h * n:(h + 1) * n].reshape(spec.dim, spec.dstate), ref,
                                       rtol=1e-11, atol=1e-14)


def test_group_mapping(orc):
    """Only heads of group g* = h // heads_per_group see a nonzero B."""
    spec = ri.with_(SMALL, H=8, hpg=4, prefix=[3, 3, 3, 3])
    prob = ri.make_problem(spec, 34)
    _, _, _, d_B, _ = ri.dense_sizes(spec)
    for l in range(spec.L):
        ring = prob.Bm[l][:, :d_B].reshape(-1, spec.R, spec.G, spec.dstate)
        ring[:, :, 0, :] = 0.0   # group 0 zero, group 1 random
    _, _, ex, _ = orc.materialize(prob, want_exact=True)
    n = spec.dim * spec.dstate
    for l, b, s, d in written_pairs(prob):
        _, _, dt = ring_views(prob, l, s)
        r0 = int(prob.meta.ring_start[b])
        for h in range(spec.H):
            tot = sum(dt[(r0 + j) % spec.R, h] for j in range(3))
            decay_only = np.exp(float(prob.A[l][h]) * tot) * prob.state[l][s, h * n:(h + 1) * n]
            close = np.allclose(ex[l][d, h * n:(h + 1) * n], decay_only, rtol=1e-12)
            assert close == (h // spec.hpg == 0)


def test_composition_fp64(orc):
    """materialize(k1) then materialize(k2) from (r0+k1) mod R, reading the
    intermediate state, equals materialize(k1+k2); fp64 storage, rel 1e-12."""
    k1 = np.array([2, 3, 0, 5])
    k2 = np.array([4, 5, 6, 3])
    base = ri.with_(SMALL, state_dtype="f64", stride_pad="none")
    p_direct = ri.make_problem(ri.with_(base, prefix=list(k1 + k2)), 40)
    _, _, ex_direct, _ = orc.materialize(p_direct)

    p1 = ri.make_problem(ri.with_(base, prefix=list(k1)), 40)
    assert np.array_equal(p1.meta.src, p_direct.meta.src)
    _, _, ex1, _ = orc.materialize(p1)
    # second call: the intermediate states (in the dst slots) are the sources;
    # their ring is the original source slot's ring, copied to the dst slot.
    p2 = ri.make_problem(ri.with_(base, prefix=list(k2)), 40)
    for l in range(base.L):
        p2.state[l] = np.where(np.isnan(ex1[l]), p1.state[l], ex1[l])
        for b in range(base.B):
            s, d = p1.meta.src[l, b], p1.meta.dst[l, b]
            for arr, arr1 in ((p2.x[l], p1.x[l]), (p2.Bm[l], p1.Bm[l]), (p2.dt[l], p1.dt[l])):
                arr[d] = arr1[s]
        p2.meta.src[l], p2.meta.dst[l] = p1.meta.dst[l].copy(), p1.meta.src[l].copy()
    p2.meta.ring_start[:] = (p1.meta.ring_start + k1) % base.R
    _, _, ex2, _ = orc.materialize(p2)
    n = base.H * base.dim * base.dstate
    for l in range(base.L):
        for b in range(base.B):
            got = ex2[l][p1.meta.src[l, b], :n]
            ref = ex_direct[l][p1.meta.dst[l, b], :n]
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_magnitude_bounds_result(orc):
    spec = ri.with_(SMALL, prefix=[8, 4, 2, 1])
    prob = ri.make_problem(spec, 41)
    _, _, ex, mg = orc.materialize(prob, want_exact=True)
    for l in range(spec.L):
        ok = ~np.isnan(ex[l])
        assert np.all(mg[l][ok] >= np.abs(ex[l][ok]) * (1 - 1e-12))
    # with no cancellation (all terms nonnegative) M equals |result|
    for l in range(spec.L):
        prob.state[l][:] = np.abs(prob.state[l])
        prob.x[l][:] = np.abs(prob.x[l])
        prob.Bm[l][:] = np.abs(prob.Bm[l])
    _, _, ex, mg = orc.materialize(prob, want_exact=True)
    for l in range(spec.L):
        ok = ~np.isnan(ex[l])
        np.testing.assert_allclose(mg[l][ok], ex[l][ok], rtol=1e-12)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "i8", "f8e4m3"])
def test_encoded_result_within_one_quantum(orc, dtype):
    """Stored codes (times the new scale) reconstruct the fp64 result within
    one grid step of the format at that value."""
    spec = ri.with_(SMALL, state_dtype=dtype, input_dtype="bf16", prefix=[3, 8, 1, 5])
    prob = ri.make_problem(spec, 42)
    st, sc, ex, _ = orc.materialize(prob, want_exact=True)
    n = spec.H * spec.dim * spec.dstate
    for l, b, s, d in written_pairs(prob):
        deq = orc.decode(dtype, st[l][d, :n]).reshape(spec.H, spec.dim, spec.dstate)
        ref = ex[l][d, :n].reshape(spec.H, spec.dim, spec.dstate)
        if ri.one_byte(dtype):
            scale = sc[l][d, :spec.H * spec.dim].reshape(spec.H, spec.dim, 1).astype(np.float64)
            rowmax = np.abs(ref).max(axis=-1, keepdims=True)
            np.testing.assert_allclose(scale, rowmax / ri.QMAX[dtype], rtol=1e-6)
            deq = deq * scale
            t = np.abs(ref) / scale
            if dtype == "i8":
                step = scale
            else:
                step = 2.0 ** (np.maximum(np.floor(np.log2(np.maximum(t, 2.0**-9))), -6) - 3) * scale
        else:
            mant, emin = (7, -126) if dtype == "bf16" else (10, -14)   # subnormal spacing below 2^emin
            step = 2.0 ** (np.maximum(np.floor(np.log2(np.maximum(np.abs(ref), 1e-300))), emin) - mant)
        assert np.all(np.abs(deq - ref) <= step * 1.0001)

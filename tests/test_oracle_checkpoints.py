"""The oracle's multi-checkpoint materialize pinned to the mathematics.

Each checkpoint is the single-checkpoint operation (flashinfer.mamba.
replayssm_materialize, Summary and Notes) with its own destination and prefix
tables, all reading the state as it was before the call; a destination may be
the source slot (the in-place flush of the pull-request page's Description).
Pins that do not reuse the oracle's own arithmetic: with x = 0 every
checkpoint is pure decay exp(A sum_{j<k_c} dt_j) S0 of the ORIGINAL source;
with A = 0 and S0 = 0 it is the product X^T diag(dt) B over its first k_c
tokens; applying k1 then k2 - k1 tokens to checkpoint k1 gives checkpoint k2
(the recurrence composes); a zero prefix copies bytes; a pad destination and
every slot no checkpoint names keep their bytes.
"""
import numpy as np
import pytest

import rssm_inputs as ri

SPEC = ri.Spec("ck_small", L=2, B=4, H=4, hpg=2, dim=8, dstate=16, R=8, W=8,
               state_dtype="f32", input_dtype="f32", k_lo=1, k_hi=8, slots=20, ring_slots=20,
               slot_mode="perm", stride_pad="per_layer")


def views(prob, l, slot):
    import oracle
    s = prob.spec
    _, _, d_x, d_B, d_dt = ri.dense_sizes(s)
    x = oracle.decode(s.input_dtype, prob.x[l][slot, :d_x]).reshape(s.R, s.H, s.dim)
    B = oracle.decode(s.input_dtype, prob.Bm[l][slot, :d_B]).reshape(s.R, s.G, s.dstate)
    dt = prob.dt[l][slot, :d_dt].astype(np.float64).reshape(s.R, s.H)
    return x, B, dt


def live(prob, dst, pre):
    """(c, l, b, src, dst, k) of every checkpoint write the call makes."""
    m, pad = prob.meta, prob.spec.pad_slot_id
    out = []
    for i in range(prob.spec.B):
        b = int(m.active[i])
        if b == -1:
            break
        for l in range(prob.spec.L):
            s = int(m.src[l, b])
            for c in range(dst.shape[0]):
                d = int(dst[c, l, b])
                if s != pad and d != pad:
                    out.append((c, l, b, s, d, int(pre[c, b])))
    return out


@pytest.mark.parametrize("in_place", [False, True])
def test_pure_decay_reads_the_original_source(orc, in_place):
    prob = ri.make_problem(SPEC, 50)
    for l in range(SPEC.L):
        prob.x[l][:] = 0.0
    dst, pre = ri.make_checkpoints(SPEC, prob.meta, 51, 3, in_place=in_place)
    state0 = [a.copy() for a in prob.state]
    _, _, ex, _ = orc.materialize_checkpoints(prob, list(dst), list(pre), want_exact=True)
    n = SPEC.dim * SPEC.dstate
    rows = live(prob, dst, pre)
    assert len({r[0] for r in rows}) == 3
    for c, l, b, s, d, k in rows:
        _, _, dt = views(prob, l, s)
        r0 = int(prob.meta.ring_start[b])
        for h in range(SPEC.H):
            tot = sum(dt[(r0 + j) % SPEC.R, h] for j in range(k))
            ref = np.exp(float(prob.A[l][h]) * tot) * state0[l][s, h * n:(h + 1) * n].astype(np.float64)
            np.testing.assert_allclose(ex[l][d, h * n:(h + 1) * n], ref, rtol=1e-12)


def test_gemm_per_checkpoint(orc):
    prob = ri.make_problem(SPEC, 52)
    for l in range(SPEC.L):
        prob.A[l][:] = 0.0
        prob.state[l][:] = 0.0
    dst, pre = ri.make_checkpoints(SPEC, prob.meta, 53, 4, dup_frac=0.25)
    _, _, ex, _ = orc.materialize_checkpoints(prob, list(dst), list(pre), want_exact=True)
    n = SPEC.dim * SPEC.dstate
    for c, l, b, s, d, k in live(prob, dst, pre):
        x, B, dt = views(prob, l, s)
        r0 = int(prob.meta.ring_start[b])
        es = [(r0 + j) % SPEC.R for j in range(k)]
        for h in range(SPEC.H):
            if k == 0:
                ref = np.zeros((SPEC.dim, SPEC.dstate))
            else:
                X = np.stack([x[e, h] for e in es])
                Bk = np.stack([B[e, h // SPEC.hpg] for e in es])
                ref = X.T @ np.diag([dt[e, h] for e in es]) @ Bk
            got = ex[l][d, h * n:(h + 1) * n].reshape(SPEC.dim, SPEC.dstate)
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_composition_across_checkpoints(orc):
    """Checkpoint k1 advanced by k2 - k1 ring entries equals checkpoint k2
    (fp64 storage; both checkpoints from one call)."""
    base = ri.with_(SPEC, state_dtype="f64", stride_pad="none", prefix=[1, 3, 2, 0])
    prob = ri.make_problem(base, 54)
    k1 = np.asarray(base.prefix, np.int32)
    k2 = np.array([5, 8, 2, 6], np.int32)
    dst, _ = ri.make_checkpoints(base, prob.meta, 55, 2)
    pre = np.stack([k1, k2])
    st, _, _, _ = orc.materialize_checkpoints(prob, list(dst), list(pre))
    # second call: the k1 checkpoints are the sources; their ring is the
    # original source slot's ring, copied into the checkpoint's slot
    p2 = ri.make_problem(ri.with_(base, prefix=list(k2 - k1)), 54)
    for l in range(base.L):
        p2.state[l] = st[l].copy()
        for b in range(base.B):
            s, d = prob.meta.src[l, b], dst[0, l, b]
            for arr, arr1 in ((p2.x[l], prob.x[l]), (p2.Bm[l], prob.Bm[l]), (p2.dt[l], prob.dt[l])):
                arr[d] = arr1[s]
        p2.meta.src[l] = dst[0, l]
        p2.meta.dst[l] = dst[1, l] + 0  # overwritten below with free slots
    p2.meta.ring_start[:] = (prob.meta.ring_start + k1) % base.R
    # write the advanced states to the original source slots (free in p2)
    for l in range(base.L):
        p2.meta.dst[l] = prob.meta.src[l]
    st2, _, _, _ = orc.materialize(p2)
    n = base.H * base.dim * base.dstate
    for l in range(base.L):
        for b in range(base.B):
            got = st2[l][prob.meta.src[l, b], :n]
            ref = st[l][dst[1, l, b], :n]
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("dtype", ["bf16", "i8", "f8e4m3"])
def test_zero_prefix_pad_and_untouched_slots(orc, dtype):
    spec = ri.with_(SPEC, state_dtype=dtype, input_dtype="bf16" if dtype != "bf16" else "bf16",
                    B=6, slots=30, ring_slots=30, n_active=5, pad_frac=0.1)
    prob = ri.make_problem(spec, 56)
    dst, pre = ri.make_checkpoints(spec, prob.meta, 57, 3, in_place=True, k0_frac=0.5, pad_frac=0.2)
    st, sc, _, _ = orc.materialize_checkpoints(prob, list(dst), list(pre))
    n, ns = spec.H * spec.dim * spec.dstate, spec.H * spec.dim
    rows = live(prob, dst, pre)
    assert any(k == 0 for *_, k in rows) and any(k > 0 for *_, k in rows)
    written = [np.zeros(a.shape, bool) for a in prob.state]
    swritten = [np.zeros(a.shape, bool) for a in prob.scale] if prob.scale else None
    for c, l, b, s, d, k in rows:
        written[l][d, :n] = True
        if swritten:
            swritten[l][d, :ns] = True
        if k == 0:
            assert np.array_equal(st[l][d, :n].view(np.uint8), prob.state[l][s, :n].view(np.uint8))
            if sc:
                assert np.array_equal(sc[l][d, :ns].view(np.uint32), prob.scale[l][s, :ns].view(np.uint32))
    for l in range(spec.L):
        assert np.array_equal(st[l][~written[l]].view(np.uint8), prob.state[l][~written[l]].view(np.uint8))
        if sc:
            assert np.array_equal(sc[l][~swritten[l]].view(np.uint32), prob.scale[l][~swritten[l]].view(np.uint32))
    # pads of checkpoints >= 1 were drawn, and their slots were not written
    assert (dst[1:] == spec.pad_slot_id).any()

"""The decode-step oracle pinned to what the pages and the mathematics fix.

The pages fix only that a checkpoint plus its ring stands for the current
state (flashinfer.mamba.replayssm_materialize, Summary) and that decode
appends to the ring (the pull request's Description).  The readout pins are
independent of the decode oracle's arithmetic: with a one-hot C_t the output
is one column of the state after n + t + 1 ring entries, which the
materialize oracle (pinned on its own) computes from the ring the step
appended to; with C = 0 it is D x silu(z); softplus matches numpy's
logaddexp; the appended bytes sit at entries (ring_start + n + t) mod R and
nothing else moves.
"""
import numpy as np
import pytest

import rssm_inputs as ri

SMALL = ri.SsuSpec("ssu_pin", B=4, H=4, hpg=2, dim=8, dstate=16, R=8, T=3, state_dtype="f32", input_dtype="f32",
                   pad_frac=0.25)


def live(prob):
    return [b for b in range(prob.spec.B) if prob.slots[b] != prob.spec.pad_slot_id]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_hot_readout_is_the_materialized_state(orc, dtype):
    spec = ri.with_(SMALL, state_dtype=dtype, input_dtype=dtype, has_D=False, has_z=False, pad_frac=0.0)
    prob = ri.make_ssu_problem(spec, 70)
    cols = np.random.default_rng(71).integers(0, spec.dstate, size=(spec.B, spec.T, spec.G))
    one = np.zeros((spec.B, spec.T, spec.G, spec.dstate), np.float32)
    for b in range(spec.B):
        for t in range(spec.T):
            for g in range(spec.G):
                one[b, t, g, cols[b, t, g]] = 1.0
    prob.C_new = ri._to_storage(one, dtype)
    xr, Br, dtr, y, _, _ = orc.ssu_decode(prob)
    # the materialize oracle on the appended rings, prefix n + t + 1 from the checkpoint slot
    pools = prob.pools
    for t in range(spec.T):
        mp = ri.make_problem(ri.with_(spec.pools(), prefix=list(prob.num_buffered + t + 1)), 70)
        mp.state, mp.x, mp.Bm, mp.dt = pools.state, [xr], [Br], [dtr]
        mp.A = [prob.A]
        mp.meta.src[0] = prob.slots
        mp.meta.ring_start[:] = prob.ring_start
        mp.meta.active[:] = np.arange(spec.B)
        _, _, ex, _ = orc.materialize(mp, want_exact=True)
        n = spec.H * spec.dim * spec.dstate
        for b in range(spec.B):
            S = ex[0][mp.meta.dst[0, b], :n].reshape(spec.H, spec.dim, spec.dstate)
            for h in range(spec.H):
                want = S[h, :, cols[b, t, h // spec.hpg]]
                np.testing.assert_allclose(y[b, t, h], want, rtol=1e-6, atol=1e-9)


def test_zero_C_leaves_gated_skip(orc):
    prob = ri.make_ssu_problem(SMALL, 72)
    prob.C_new[:] = 0
    _, _, _, y, _, _ = orc.ssu_decode(prob)
    x = prob.x_new.astype(np.float64)
    z = prob.z.astype(np.float64)
    want = prob.D.astype(np.float64)[None, None, :, None] * x * (z / (1.0 + np.exp(-z)))
    for b in live(prob):
        np.testing.assert_allclose(y[b], want[b], rtol=1e-13)


def test_readout_is_linear_in_C(orc):
    spec = ri.with_(SMALL, has_D=False)
    p1, p2, p12 = (ri.make_ssu_problem(spec, 73) for _ in range(3))
    rng = np.random.default_rng(74)
    # bf16-representable draws, so that c1 + c2 is exact in fp32
    c1 = ri._to_storage(rng.standard_normal(p1.C_new.shape).astype(np.float32), "bf16")
    c2 = ri._to_storage(rng.standard_normal(p1.C_new.shape).astype(np.float32), "bf16")
    c1 = (c1.astype(np.uint32) << 16).view(np.float32)
    c2 = (c2.astype(np.uint32) << 16).view(np.float32)
    c12 = c1 + c2
    exact = c12.astype(np.float64) == c1.astype(np.float64) + c2.astype(np.float64)
    c1, c2 = np.where(exact, c1, 0).astype(np.float32), np.where(exact, c2, 0).astype(np.float32)
    p1.C_new, p2.C_new, p12.C_new = c1, c2, c1 + c2
    y1, y2, y12 = (orc.ssu_decode(p)[3] for p in (p1, p2, p12))
    for b in live(p1):
        np.testing.assert_allclose(y12[b], y1[b] + y2[b], rtol=1e-9, atol=1e-9)


def test_softplus_and_appended_entries(orc):
    prob = ri.make_ssu_problem(ri.with_(SMALL, buffered=[0, 5, 2, 4]), 75)
    spec, pools = prob.spec, prob.pools
    xr, Br, dtr, y, _, dte = orc.ssu_decode(prob)
    want_dt = np.logaddexp(0.0, prob.dt_new.astype(np.float64) + prob.dt_bias.astype(np.float64)[None, None, :])
    m = pools.meta
    dH, dG = spec.H * spec.dim, spec.G * spec.dstate
    changed_x = np.zeros(xr.shape, bool)
    changed_B = np.zeros(Br.shape, bool)
    changed_dt = np.zeros(dtr.shape, bool)
    for b in range(spec.B):
        s = int(prob.slots[b])
        if s == spec.pad_slot_id:
            assert np.isnan(y[b]).all() and np.isnan(dte[b]).all()
            continue
        np.testing.assert_allclose(dte[b], want_dt[b], rtol=1e-14)
        for t in range(spec.T):
            e = (int(prob.ring_start[b]) + int(prob.num_buffered[b]) + t) % spec.R
            xs = slice(e * dH, (e + 1) * dH)
            assert np.array_equal(xr[s, xs], prob.x_new[b, t].reshape(-1))
            Bs = slice(e * dG, (e + 1) * dG)
            assert np.array_equal(Br[s, Bs], prob.B_new[b, t].reshape(-1))
            ds_ = slice(e * spec.H, (e + 1) * spec.H)
            assert np.array_equal(dtr[s, ds_], want_dt[b, t].astype(np.float32))
            changed_x[s, xs] = changed_B[s, Bs] = changed_dt[s, ds_] = True
    assert np.array_equal(xr[~changed_x], pools.x[0][~changed_x])
    assert np.array_equal(Br[~changed_B], pools.Bm[0][~changed_B])
    assert np.array_equal(dtr[~changed_dt], pools.dt[0][~changed_dt])
    assert m.x_stride[0] > dH  # the stride gap is part of what must not move

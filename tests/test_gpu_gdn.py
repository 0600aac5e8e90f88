"""GPU parity of the gated-delta-rule commit (rssm_gdn_commit, through the
C ABI) against the CPU oracle.

Tolerance, from the arithmetic: per token the fp32 path rounds the key
normalisation (a 128-term sum of squares, a root and a division: a few ulps
per key element), the dot product S k (8 fused multiply-adds per lane and a
16-lane tree: gamma_12 of sum |S||k|) and the update (two roundings of
|S'|).  Each is at most ~20 u of the magnitude bound M that the oracle
carries (u = 2^-24), and the update is non-expanding (exp(g) <= 1 and
|I - beta k k^T| <= 1 for unit keys and beta in [0, 1]), so errors of
earlier tokens do not grow: after n <= 16 tokens |gpu - exact| <= 320 u M
< 2e-5 M.  Everything the call must not write is compared bit for bit.
"""
import sys

import numpy as np
import pytest

import rssm_inputs as ri

pytestmark = pytest.mark.gpu
TOL = 2e-5


def say(*a):
    print("[gpu-gdn]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import replayssm_persistent_rssm_amd as rp  # noqa: F401  (fails loudly if the library is missing)
    return torch.device("cuda:0")


def upload(prob, dev):
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    d = dict(state=t(prob.state), rawv=bf(prob.rawv), rawk=bf(prob.rawk), g=t(prob.g), beta=t(prob.beta),
             idx=t(prob.state_indices.astype(np.int32)), acc=t(prob.accept_lens.astype(np.int32)),
             tidx=t(prob.track_state_indices.astype(np.int32)) if prob.track_state_indices is not None else None,
             tstep=t(prob.track_steps.astype(np.int32)) if prob.track_steps is not None else None)
    return d


def run(prob, dev, max_workgroups=0):
    import torch
    import replayssm_persistent_rssm_amd as rp
    d = upload(prob, dev)
    rp.rssm_gdn_commit(d["state"], d["rawv"], d["rawk"], d["g"], d["beta"], d["idx"], d["acc"],
                       track_state_indices=d["tidx"], track_steps=d["tstep"], use_qk_l2norm=prob.spec.use_l2norm,
                       null_block_id=prob.spec.null_block_id, max_workgroups=max_workgroups)
    torch.cuda.synchronize()
    for name, arr in (("rawv", prob.rawv), ("rawk", prob.rawk)):
        assert np.array_equal(d[name].view(torch.int16).cpu().numpy().view(np.uint16), arr), f"{name} changed"
    assert np.array_equal(d["g"].cpu().numpy(), prob.g) and np.array_equal(d["beta"].cpu().numpy(), prob.beta)
    return d["state"].cpu().numpy()


def check(prob, got, what=""):
    import oracle
    _, ex, mg = oracle.gdn_commit(prob, want_exact=True)
    w = ~np.isnan(ex)
    assert np.array_equal(got[~w].view(np.uint32), prob.state[~w].view(np.uint32)), f"{what}: untouched bytes changed"
    err = np.abs(got[w].astype(np.float64) - ex[w])
    ratio = err / np.maximum(mg[w], 1e-300)
    say(what, "written elements", int(w.sum()), "max |gpu-exact|/M", float(ratio.max()) if w.any() else 0.0)
    assert (err <= TOL * mg[w]).all(), f"{what}: {int((err > TOL * mg[w]).sum())} elements beyond {TOL}*M"
    return w


@pytest.mark.parametrize("seed", [70, 71])
def test_small_workload(dev, seed):
    spec = ri.GDN_CONFIGS["gdn_small"]
    prob = ri.make_gdn_problem(spec, seed)
    say("gdn_small seed", seed, "accept", prob.accept_lens.tolist(), "track steps", prob.track_steps.tolist())
    w = check(prob, run(prob, dev), f"gdn_small/{seed}")
    assert w.any()


@pytest.mark.parametrize("kw", [
    dict(track=False),
    dict(use_l2norm=False),
    dict(null_block_id=3, null_frac=0.3),
    dict(T=16, HV=3, H=3, accept=[16, 9, 0, 1, 15, 16]),
    dict(T=3, HV=8, H=1),
    dict(T=5, accept=[5, 5, 5, 5, 5, 5], zero_frac=0.0, null_frac=0.0),
    dict(L=80, HV=2, H=1),   # more layers than a wavefront has lanes
])
def test_variants(dev, kw):
    spec = ri.with_(ri.GDN_CONFIGS["gdn_small"], **kw)
    prob = ri.make_gdn_problem(spec, 72)
    if not spec.use_l2norm:
        # unnormalised keys scaled to |k|^2 < 2, so the update stays non-expanding
        k = (prob.rawk.astype(np.uint32) << 16).view(np.float32) * np.float32(1.0 / 16)
        prob.rawk = ri._bf16_codes(k)
    say("variant", kw)
    check(prob, run(prob, dev), str(kw))


def test_out_of_range_metadata_guards(dev):
    """Device metadata outside its documented range is not checked (as on the
    page); the kernel guards against faults instead: a state slot at or past
    `slots` is skipped, accepted counts are clamped to [0, T], and a track
    slot at or past `slots` leaves the tracked step unwritten.  The result
    must equal the oracle's on metadata sanitised that way (the oracle itself
    rejects such values)."""
    import copy
    spec = ri.with_(ri.GDN_CONFIGS["gdn_small"], B=8, slots=24, null_frac=0.0, zero_frac=0.0)
    bad = ri.make_gdn_problem(spec, 74)
    T, S, null = spec.T, spec.slots, spec.null_block_id
    bad.accept_lens = bad.accept_lens.copy()
    bad.state_indices = bad.state_indices.copy()
    bad.track_state_indices = bad.track_state_indices.copy()
    bad.track_steps = bad.track_steps.copy()
    bad.accept_lens[0] = T + 5                # clamped to T
    bad.accept_lens[1] = -3                   # clamped to 0: nothing committed
    bad.state_indices[2] = S + 4              # out of range: skipped
    bad.track_state_indices[3] = S + 7        # out of range: tracked step not written
    bad.track_steps[3] = 0
    sane = copy.copy(bad)
    sane.accept_lens = np.clip(bad.accept_lens, 0, T).astype(bad.accept_lens.dtype)
    sane.state_indices = np.where(bad.state_indices >= S, null, bad.state_indices).astype(bad.state_indices.dtype)
    sane.track_state_indices = np.where(bad.track_state_indices >= S, null,
                                        bad.track_state_indices).astype(bad.track_state_indices.dtype)
    say("out-of-range metadata")
    check(sane, run(bad, dev), "out-of-range metadata")


def test_nothing_to_commit(dev):
    spec = ri.with_(ri.GDN_CONFIGS["gdn_small"], accept=[0] * 6)
    prob = ri.make_gdn_problem(spec, 73)
    got = run(prob, dev)
    assert np.array_equal(got.view(np.uint32), prob.state.view(np.uint32))


def test_grid_invariance(dev):
    """Each work item's arithmetic is independent of the launch shape: the
    bytes are identical for any grid."""
    spec = ri.with_(ri.GDN_CONFIGS["gdn_small"], B=9, slots=24, HV=8, H=4)
    prob = ri.make_gdn_problem(spec, 74)
    ref = run(prob, dev)
    for g in (1, 3, 37):
        assert np.array_equal(run(prob, dev, max_workgroups=g).view(np.uint32), ref.view(np.uint32)), g


@pytest.mark.parametrize("null_frac", [0.5, 1.0])
def test_null_requests_many_tiles_per_wave(dev, null_frac):
    """Null slots and zero accepted counts mixed with live requests (or every
    request null) on grids of 1-2 workgroups: each wavefront deals up to 192
    tiles, so it tests their liveness in several batches of 64 and skips the
    dead ones; the default grid as well."""
    spec = ri.with_(ri.GDN_CONFIGS["gdn_small"], B=24, L=4, HV=8, H=4, slots=56, null_frac=null_frac,
                    zero_frac=0.2 if null_frac < 1 else 0.0)
    prob = ri.make_gdn_problem(spec, 75)
    for g in (1, 2, 0):
        say("null_frac", null_frac, "grid", g)
        got = run(prob, dev, max_workgroups=g)
        if null_frac == 1.0:
            assert np.array_equal(got.view(np.uint32), prob.state.view(np.uint32)), "an all-null call wrote"
        else:
            assert check(prob, got, f"null_frac {null_frac} grid {g}").any()


def test_full_size_sampled(dev):
    """gdn_large at full size, in the launch the benchmark times: sampled
    tiles against the oracle (the states are copied before the in-place
    commit), and slots that are neither live nor tracked keep their fill."""
    import torch
    import oracle
    import replayssm_persistent_rssm_amd as rp
    spec = ri.GDN_CONFIGS["gdn_large"]
    seed = 1010
    say("gdn_large full size, seed", seed)
    dp = ri.make_gdn_device_problem(spec, seed, dev)
    idx, acc, tidx, tstep = dp.state_indices, dp.accept_lens, dp.track_state_indices, dp.track_steps
    rng = np.random.default_rng(seed)
    live = [b for b in range(spec.B) if idx[b] > spec.null_block_id and acc[b] > 0]
    picks = [(live[0], 0, 0), (live[-1], spec.L - 1, spec.HV - 1)]
    picks += [(int(rng.choice(live)), int(rng.integers(spec.L)), int(rng.integers(spec.HV))) for _ in range(20)]
    tracked = [b for b in live if tidx[b] > spec.null_block_id and 0 <= tstep[b] < acc[b]]
    picks += [(int(b), int(rng.integers(spec.L)), int(rng.integers(spec.HV))) for b in tracked[:4]]
    before = {(b, l, h): dp.state[l, int(idx[b]), h].cpu().numpy().copy() for b, l, h in picks}
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)  # noqa: E731
    rp.rssm_gdn_commit(dp.state, dp.rawv, dp.rawk, dp.g, dp.beta, i32(idx), i32(acc),
                       track_state_indices=i32(tidx), track_steps=i32(tstep), null_block_id=spec.null_block_id)
    torch.cuda.synchronize()
    group = spec.HV // spec.H
    worst = 0.0
    for b, l, h in picks:
        s = int(idx[b])
        kwin = dp.rawk[l, s, h // group].view(torch.int16).cpu().numpy().view(np.uint16)
        vwin = dp.rawv[l, s, h].view(torch.int16).cpu().numpy().view(np.uint16)
        fin, mfin, trk, mtrk = oracle.gdn_tile(spec, before[(b, l, h)], kwin, vwin, dp.g[l, s, h].cpu().numpy(),
                                               dp.beta[l, s, h].cpu().numpy(), int(acc[b]), int(tstep[b]))
        got = dp.state[l, s, h].cpu().numpy().astype(np.float64)
        err = np.abs(got - fin)
        worst = max(worst, float((err / mfin).max()))
        assert (err <= TOL * mfin).all(), (b, l, h)
        if trk is not None and tidx[b] > spec.null_block_id:
            gt = dp.state[l, int(tidx[b]), h].cpu().numpy().astype(np.float64)
            assert (np.abs(gt - trk) <= TOL * mtrk).all(), ("track", b, l, h)
    say("full size: worst |gpu-exact|/M", worst)
    # a slot no request names keeps its fill bytes
    named = set(int(v) for v in idx) | set(int(v) for v in tidx)
    free = [s for s in range(spec.slots) if s not in named]
    if free:
        t = dp.state[0, free[:4]].view(torch.uint8)
        assert bool((t == 0xA5).all().item())
    del dp
    torch.cuda.empty_cache()

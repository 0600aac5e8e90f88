"""GPU parity of the ReplaySSM decode step (rssm_ssu_decode, through the C
ABI) against the CPU oracle.

Tolerance, from the arithmetic: the kernel evaluates
y = Dec (S_0 . C) + sum_j w_j (B_j . C) x_j + D x in fp32.  Each dot product
is 8 fused multiply-adds per lane and a 16-lane tree (at most 12 roundings
of the sum of absolute products); a decay is exp of a rounded product (a few
ulps), Dec and the weights are products of at most 16 of them (at most ~64 u
relative); a new token's dt is an fp32 softplus (a few ulps; the oracle keeps
it in fp64); the final sum has at most 20 terms.  Every error term is a
relative error of a product whose absolute value the oracle's magnitude bound
M_y covers (M_y bounds sum_c |S[r][c]| |C[c]| + |D x| along the recurrence),
so |gpu - exact| <= ~150 u M_y < 1e-5 M_y (u = 2^-24); the test allows
2e-5 M_y.  The appended x and B bytes and every byte the call must not write
are compared bit for bit.  An appended dt is an fp32 softplus of the exact
sum raw + bias (kept as a hi + lo pair): an exp, a product, a log1p and an
add, each off by at most ~2 ulps of its result, so the test allows 8 ulps of
the fp64 value (numpy's fp32 evaluation of the same formula reaches 3.7).
"""
import sys

import numpy as np
import pytest

import rssm_inputs as ri

pytestmark = pytest.mark.gpu
TOL = 2e-5
DT_ULPS = 8


def say(*a):
    print("[gpu-ssu]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import replayssm_persistent_rssm_amd as rp  # noqa: F401  (fails loudly if the library is missing)
    return torch.device("cuda:0")


def run(prob, dev, max_workgroups=0):
    import torch
    import rssm_harness as hx
    d = ri.ssu_to_device(prob, dev)
    state_before = d.state.clone()
    hx.ssu_call(d, max_workgroups=max_workgroups)
    torch.cuda.synchronize()
    assert torch.equal(d.state.view(torch.uint8), state_before.view(torch.uint8)), "the checkpoint was written"
    return hx.ssu_download(d)


def check(prob, got, what=""):
    import oracle
    spec = prob.spec
    xr_g, Br_g, dtr_g, y_g = got
    xr, Br, dtr, y, ym, dte = oracle.ssu_decode(prob)
    assert np.array_equal(xr_g.view(np.uint8), xr.view(np.uint8)), f"{what}: x ring differs"
    assert np.array_equal(Br_g.view(np.uint8), Br.view(np.uint8)), f"{what}: B ring differs"
    # dt ring: bytes identical except the appended entries, which are within DT_ULPS of the fp64 value
    appended = np.zeros(dtr.shape, bool)
    for b in range(spec.B):
        s = int(prob.slots[b])
        if s == spec.pad_slot_id:
            continue
        for t in range(spec.T):
            e = (int(prob.ring_start[b]) + int(prob.num_buffered[b]) + t) % spec.R
            appended[s, e * spec.H:(e + 1) * spec.H] = True
            want = dte[b, t]
            ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
            err = np.abs(dtr_g[s, e * spec.H:(e + 1) * spec.H].astype(np.float64) - want)
            assert (err <= DT_ULPS * ulp).all(), f"{what}: appended dt of request {b} token {t}"
    assert np.array_equal(dtr_g[~appended].view(np.uint32), dtr[~appended].view(np.uint32)), f"{what}: dt ring"
    live = np.array([int(s) != spec.pad_slot_id for s in prob.slots])
    if (~live).any():
        assert np.isnan(y_g[~live]).all(), f"{what}: padded requests' outputs were written"
    err = np.abs(y_g[live].astype(np.float64) - y[live])
    bound = TOL * ym[live]
    ratio = err / np.maximum(ym[live], 1e-300)
    say(what, "live requests", int(live.sum()), "max |gpu-exact|/M", float(ratio.max()) if live.any() else 0.0)
    assert (err <= bound).all(), f"{what}: {int((err > bound).sum())} outputs beyond {TOL}*M"


@pytest.mark.parametrize("seed", [80, 81])
def test_small_workload(dev, seed):
    spec = ri.SSU_CONFIGS["ssu_small"]
    prob = ri.make_ssu_problem(spec, seed)
    say("ssu_small seed", seed, "slots", prob.slots.tolist(), "buffered", prob.num_buffered.tolist(),
        "ring_start", prob.ring_start.tolist())
    check(prob, run(prob, dev), f"ssu_small/{seed}")


VARIANTS = [
    dict(state_dtype="f32", input_dtype="f32"),
    dict(state_dtype="f16", input_dtype="f16"),
    dict(state_dtype="bf16", input_dtype="f32"),
    dict(state_dtype="f32", input_dtype="bf16"),
    dict(state_dtype="f16", input_dtype="bf16"),
    dict(state_dtype="f32", input_dtype="f16"),
    dict(state_dtype="bf16", input_dtype="f16", T=6),
    dict(T=1),
    dict(T=3, buffered=[13, 0, 7, 12, 1]),
    dict(T=5),
    dict(T=8, buffered=[8, 0, 3, 8, 5]),
    dict(has_z=False, has_D=False),
    dict(has_bias=False, dt_softplus=False),
    dict(buffered=[12, 12, 12, 12, 12]),
    dict(buffered=[0, 0, 0, 0, 0]),
    dict(hpg=1),
    dict(hpg=8),
    dict(R=20, buffered=[12, 3, 0, 9, 11]),
    dict(R=5, T=2, buffered=[3, 0, 1, 2, 3]),
    dict(B=37, H=16, hpg=4, pad_frac=0.1),
    dict(pad_frac=1.0),
]


@pytest.mark.parametrize("kw", VARIANTS, ids=[str(v) for v in VARIANTS])
def test_variants(dev, kw):
    spec = ri.with_(ri.SSU_CONFIGS["ssu_small"], **kw)
    prob = ri.make_ssu_problem(spec, 82)
    say("variant", kw, "buffered", prob.num_buffered.tolist())
    check(prob, run(prob, dev), str(kw))


def test_out_of_range_metadata_guards(dev):
    """Device metadata outside its documented range is not checked; the
    kernel guards against faults instead: a slot outside [0, num_slots) is
    skipped (its outputs stay unwritten), ring_start is taken modulo R and
    num_buffered is clamped to [0, min(16, R) - T].  The result must equal
    the oracle's on metadata sanitised that way (the oracle itself rejects
    such values)."""
    import copy
    spec = ri.with_(ri.SSU_CONFIGS["ssu_small"], B=6, pad_frac=0.0)
    bad = ri.make_ssu_problem(spec, 86)
    R, T, pad = spec.R, spec.T, spec.pad_slot_id
    n_slots = bad.pools.meta.slots
    for name in ("slots", "ring_start", "num_buffered"):
        setattr(bad, name, getattr(bad, name).copy())
    bad.num_buffered[0] = 30                  # clamped to min(16, R) - T
    bad.num_buffered[1] = -2                  # clamped to 0
    bad.ring_start[2] = -5                    # taken modulo R
    bad.ring_start[3] = 2 * R + 3
    bad.slots[4] = n_slots + 2                # out of range: skipped
    sane = copy.copy(bad)
    sane.num_buffered = np.clip(bad.num_buffered, 0, min(16, R) - T).astype(np.int32)
    sane.ring_start = np.mod(bad.ring_start, R).astype(np.int32)
    sane.slots = np.where((bad.slots < 0) | (bad.slots >= n_slots), pad, bad.slots).astype(np.int32)
    say("out-of-range metadata")
    check(sane, run(bad, dev), "out-of-range metadata")


def test_grid_invariance(dev):
    """Each (request, head) item's arithmetic is independent of the launch
    shape: outputs and rings are identical bytes for any grid."""
    spec = ri.with_(ri.SSU_CONFIGS["ssu_small"], B=9, H=16, hpg=4, pad_frac=0.2)
    prob = ri.make_ssu_problem(spec, 83)
    ref = run(prob, dev)
    for g in (1, 3, 37):
        got = run(prob, dev, max_workgroups=g)
        for a, b in zip(got, ref):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), g


def test_xcd_block_order_runs_and_tail(dev):
    """The kernel renumbers workgroups within each full run of 64 so that one
    XCD's eight take consecutive items; the tail keeps launch order.  368
    items give a default grid of 92 workgroups (one run and a tail of 28):
    against the oracle, and byte-identical at grids of 64 (one run), 128 (two),
    130 (two and a tail) and 1."""
    spec = ri.with_(ri.SSU_CONFIGS["ssu_small"], B=23, H=16, hpg=8, pad_frac=0.1)
    prob = ri.make_ssu_problem(spec, 87)
    say("block order: B=23 H=16, default grid 92")
    ref = run(prob, dev)
    check(prob, ref, "block order, default grid")
    for g in (64, 128, 130, 1):
        got = run(prob, dev, max_workgroups=g)
        for a, b in zip(got, ref):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), g


def test_empty_batch(dev):
    import torch
    import replayssm_persistent_rssm_amd as rp
    spec = ri.SSU_CONFIGS["ssu_small"]
    prob = ri.make_ssu_problem(spec, 84)
    d = ri.ssu_to_device(prob, dev)
    e = lambda *s, dt=d.x_new.dtype: torch.empty(s, dtype=dt, device=dev)  # noqa: E731
    x_ring_before = d.x_ring.clone()
    rp.rssm_ssu_decode(d.state, d.x_ring, d.B_ring, d.dt_ring, d.A, e(0, spec.T, spec.H, spec.dim),
                       e(0, spec.T, spec.G, spec.dstate), e(0, spec.T, spec.G, spec.dstate),
                       e(0, spec.T, spec.H, dt=torch.float32), e(0, spec.T, spec.H, spec.dim, dt=torch.float32),
                       e(0, dt=torch.int32), e(0, dt=torch.int32), e(0, dt=torch.int32), ring_buffer_len=spec.R)
    torch.cuda.synchronize()
    assert torch.equal(d.x_ring, x_ring_before)


def test_binding_rejects_bad_tensors(dev):
    import torch
    import replayssm_persistent_rssm_amd as rp
    spec = ri.SSU_CONFIGS["ssu_small"]
    d = ri.ssu_to_device(ri.make_ssu_problem(spec, 85), dev)
    base = [d.state, d.x_ring, d.B_ring, d.dt_ring, d.A, d.x_new, d.B_new, d.C_new, d.dt_new, d.y, d.slots,
            d.ring_start, d.num_buffered]
    with pytest.raises(ValueError):   # y must be fp32
        bad = list(base)
        bad[9] = d.y.to(torch.bfloat16)
        rp.rssm_ssu_decode(*bad, ring_buffer_len=spec.R)
    with pytest.raises(ValueError):   # x ring in another dtype than the inputs
        bad = list(base)
        bad[1] = d.x_ring.float()
        rp.rssm_ssu_decode(*bad, ring_buffer_len=spec.R)
    with pytest.raises(rp.RssmError):   # more tokens than an instance covers
        big = ri.with_(spec, T=9, R=16, buffered=[0] * spec.B)
        d9 = ri.ssu_to_device(ri.make_ssu_problem(big, 86), dev)
        import rssm_harness as hx
        hx.ssu_call(d9)


def _host_subproblem(spec, d, picks):
    """A host problem holding only the picked requests of a device problem:
    their slots' checkpoints and rings copied back, slots renumbered."""
    import rssm_harness as hx
    sub = ri.with_(spec, B=len(picks), slots=2 * len(picks), pad_frac=0.0, buffered=None)
    prob = ri.make_ssu_problem(sub, 0)
    sl = [int(d.slots_np[b]) for b in picks]
    it, st = spec.input_dtype, spec.state_dtype
    prob.pools.state[0] = hx._host_storage(d.state[sl], st).copy()
    prob.pools.x[0] = hx._host_storage(d.x_ring[sl], it).copy()
    prob.pools.Bm[0] = hx._host_storage(d.B_ring[sl], it).copy()
    prob.pools.dt[0] = d.dt_ring[sl].cpu().numpy().copy()
    prob.slots = np.arange(len(picks), dtype=np.int32)
    prob.ring_start = d.ring_start_np[picks].copy()
    prob.num_buffered = d.num_buffered_np[picks].copy()
    prob.A = d.A.cpu().numpy()
    prob.D = d.D.cpu().numpy() if d.D is not None else None
    prob.dt_bias = d.dt_bias.cpu().numpy() if d.dt_bias is not None else None
    prob.x_new = hx._host_storage(d.x_new[picks], it).copy()
    prob.B_new = hx._host_storage(d.B_new[picks], it).copy()
    prob.C_new = hx._host_storage(d.C_new[picks], it).copy()
    prob.dt_new = d.dt_new[picks].cpu().numpy().copy()
    prob.z = hx._host_storage(d.z[picks], it).copy() if d.z is not None else None
    return prob


def test_full_size_sampled(dev):
    """ssu_large at full size, in the launch the benchmark times: sampled
    requests against the oracle (their slots copied before the call), and the
    ring bytes of the sampled slots after it."""
    import torch
    import oracle
    import rssm_harness as hx
    spec = ri.SSU_CONFIGS["ssu_large"]
    seed = 1020
    say("ssu_large full size, seed", seed)
    d = ri.make_ssu_device_problem(spec, seed, dev)
    rng = np.random.default_rng(seed)
    live = [b for b in range(spec.B) if int(d.slots_np[b]) != spec.pad_slot_id]
    nb = d.num_buffered_np
    picks = sorted(set([live[0], live[-1], int(live[int(np.argmax(nb[live]))]), int(live[int(np.argmin(nb[live]))])]
                       + [int(v) for v in rng.choice(live, size=8, replace=False)]))
    prob = _host_subproblem(spec, d, picks)
    state_sample = d.state[int(d.slots_np[picks[0]])].clone()
    hx.ssu_call(d)
    torch.cuda.synchronize()
    assert torch.equal(d.state[int(d.slots_np[picks[0]])].view(torch.int16), state_sample.view(torch.int16))
    xr, Br, dtr, y, ym, dte = oracle.ssu_decode(prob)
    sl = [int(d.slots_np[b]) for b in picks]
    it = spec.input_dtype
    assert np.array_equal(hx._host_storage(d.x_ring[sl], it), xr)
    assert np.array_equal(hx._host_storage(d.B_ring[sl], it), Br)
    y_g = d.y[picks].cpu().numpy().astype(np.float64)
    err = np.abs(y_g - y)
    say("full size: picks", picks, "worst |gpu-exact|/M", float((err / ym).max()))
    assert (err <= TOL * ym).all()
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", [90, 91])
def test_decode_flush_decode_chain(dev, seed):
    """The serving loop on the GPU: a decode step appends T tokens, an in-place
    materialize flushes all n + T buffered tokens into the checkpoint, and a
    second decode step starts from that checkpoint with an empty ring window.
    Its outputs equal the oracle's decode step run on the ORIGINAL checkpoint
    with n + T pending entries (the oracle's own appended ring) and the same
    second tokens.  fp32 state, so the flush rounds the state once to fp32,
    which the tolerance's M bound covers."""
    import copy
    import torch
    import oracle
    import rssm_harness as hx
    spec = ri.with_(ri.SSU_CONFIGS["ssu_small"], state_dtype="f32", input_dtype="f32", buffered=[3, 0, 8, 5, 1])
    p1 = ri.make_ssu_problem(spec, seed)
    p2 = ri.make_ssu_problem(spec, seed + 100)   # the second step's tokens
    T, R = spec.T, spec.R
    say("chain seed", seed, "slots", p1.slots.tolist(), "buffered", p1.num_buffered.tolist())
    # device pools shared by the three calls
    dp = hx.upload(p1.pools, dev)
    m = dp.meta
    live = np.array([int(s) != spec.pad_slot_id for s in p1.slots])
    t32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev) if a is not None else None  # noqa: E731
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)  # noqa: E731

    def step(p, ring_start, buffered):
        y = torch.full((spec.B, T, spec.H, spec.dim), float("nan"), dtype=torch.float32, device=dev)
        d = ri.SsuDeviceProblem(spec=spec, state=dp.state[0], x_ring=dp.x[0], B_ring=dp.Bm[0], dt_ring=dp.dt[0],
                                A=dp.A[0], D=t32(p.D), dt_bias=t32(p.dt_bias), x_new=t32(p.x_new), B_new=t32(p.B_new),
                                C_new=t32(p.C_new), dt_new=t32(p.dt_new), z=t32(p.z), y=y, slots=i32(p1.slots),
                                ring_start=i32(ring_start), num_buffered=i32(buffered), slots_np=p1.slots,
                                ring_start_np=ring_start, num_buffered_np=buffered)
        hx.ssu_call(d)
        return y

    step(p1, p1.ring_start, p1.num_buffered)
    # flush in place: src = dst = the request's slot, prefix n + T from its ring start
    m.src[0] = p1.slots
    m.dst[0] = p1.slots
    m.ring_start[:] = p1.ring_start
    m.prefix[:] = p1.num_buffered + T
    act = np.full(spec.B, -1, np.int32)
    act[:int(live.sum())] = np.nonzero(live)[0]
    hx.materialize(dp, hx.tables(dp, dev), active=i32(act))
    rs2 = ((p1.ring_start + p1.num_buffered + T) % R).astype(np.int32)
    y2 = step(p2, rs2, np.zeros(spec.B, np.int32)).cpu().numpy()
    torch.cuda.synchronize()

    # the oracle: the original checkpoint, its own appended ring, n + T pending, the second tokens
    xr, Br, dtr, _, _, _ = oracle.ssu_decode(p1)
    q = copy.deepcopy(p2)
    q.pools = copy.deepcopy(p1.pools)
    q.pools.x[0], q.pools.Bm[0], q.pools.dt[0] = xr, Br, dtr
    q.slots, q.ring_start, q.A = p1.slots, p1.ring_start, p1.A
    q.num_buffered = (p1.num_buffered + T).astype(np.int32)
    _, _, _, y, ym, _ = oracle.ssu_decode(q)
    err = np.abs(y2[live].astype(np.float64) - y[live])
    say("chain: max |gpu-exact|/M", float((err / np.maximum(ym[live], 1e-300)).max()))
    assert (err <= TOL * ym[live]).all()
    assert np.isnan(y2[~live]).all()

"""GPU parity of the multi-checkpoint entry point and of in-place flushes.

rssm_materialize_checkpoints writes up to four checkpoints per request from
one read of each source tile; the oracle defines each checkpoint as its own
single-checkpoint materialize from the pre-call state.  A destination may be
the source slot (in-place flush), for both entry points.
"""
import copy
import sys

import numpy as np
import pytest

import rssm_inputs as ri

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-checkpoints]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import replayssm_persistent_rssm_amd as rp  # noqa: F401  (fails loudly if the library is missing)
    return torch.device("cuda:0")


def i32(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)


def run_checkpoints(prob, dst, pre, dev, max_workgroups=0):
    import torch
    import rssm_harness as hx
    dp = hx.upload(prob, dev)
    tabs = hx.tables(dp, dev)
    call = hx.prepared_checkpoints(dp, tabs, i32(dst, dev), i32(pre, dev), max_workgroups=max_workgroups)
    call()
    torch.cuda.synchronize()
    st = hx.download(dp.state, prob.state)
    sc = hx.download(dp.scale, prob.scale) if prob.scale else None
    for got, want in zip([hx.download(dp.x, prob.x), hx.download(dp.Bm, prob.Bm), hx.download(dp.dt, prob.dt)],
                         [prob.x, prob.Bm, prob.dt]):
        for g, w in zip(got, want):
            assert np.array_equal(g.view(np.uint8), w.view(np.uint8)), "ring changed"
    return st, sc


CK = ri.Spec("ck", L=2, B=5, H=8, hpg=4, dim=64, dstate=128, R=8, W=8, k_lo=0, k_hi=8,
             slots=25, ring_slots=25, slot_mode="perm", stride_pad="per_layer", rand_seed=91, n_active=4)


@pytest.mark.parametrize("state", ["f32", "bf16", "f16", "i8", "f8e4m3"])
@pytest.mark.parametrize("rounds", [0, 10])
@pytest.mark.parametrize("n_ck,in_place", [(2, True), (3, False), (4, True)])
def test_checkpoints_against_oracle(dev, state, rounds, n_ck, in_place):
    import parity
    if state == "f32" and rounds:
        pytest.skip("fp32 state is never rounded")
    spec = ri.with_(CK, state_dtype=state, input_dtype="bf16", philox_rounds=rounds, pad_frac=0.1)
    seed = 3000 + 10 * ri.DTYPE_CODE[state] + n_ck + rounds
    prob = ri.make_problem(spec, seed)
    dst, pre = ri.make_checkpoints(spec, prob.meta, seed + 1, n_ck, in_place=in_place, k0_frac=0.2,
                                   pad_frac=0.2, dup_frac=0.2)
    say("checkpoints", state, "rounds", rounds, "n_ck", n_ck, "in_place", in_place, "seed", seed)
    st, sc = run_checkpoints(prob, dst, pre, dev)
    parity.check_checkpoints_against_oracle(prob, dst, pre, st, sc)


@pytest.mark.parametrize("H", [8, 24])
def test_checkpoints_mixed_pads_many_chunks_per_wave(dev, H):
    """Pad sources and pad checkpoint destinations mixed with live pairs on
    grids of 1-3 workgroups, so each wavefront deals many chunks and skips
    dead ones from its batched liveness test (H = 24: chunks straddle pairs)."""
    import parity
    spec = ri.with_(CK, L=6, B=24, H=H, hpg=8, dim=64, dstate=128, slots=96, ring_slots=96, n_active=22,
                    state_dtype="bf16", input_dtype="bf16", pad_frac=0.5)
    seed = 3090 + H
    prob = ri.make_problem(spec, seed)
    dst, pre = ri.make_checkpoints(spec, prob.meta, seed + 1, 3, in_place=True, k0_frac=0.2, pad_frac=0.6)
    for mw in (1, 3):
        say("checkpoints mixed pads H", H, "grid", mw, "seed", seed)
        st, sc = run_checkpoints(prob, dst, pre, dev, max_workgroups=mw)
        parity.check_checkpoints_against_oracle(prob, dst, pre, st, sc)


def test_checkpoints_window_16_wrapping_ring(dev):
    import parity
    spec = ri.with_(CK, W=16, R=5, k_lo=0, k_hi=16, state_dtype="bf16", input_dtype="f16", philox_rounds=10)
    prob = ri.make_problem(spec, 3100)
    dst, pre = ri.make_checkpoints(spec, prob.meta, 3101, 4, in_place=True, k0_frac=0.1, dup_frac=0.1)
    say("checkpoints W=16 R=5")
    st, sc = run_checkpoints(prob, dst, pre, dev)
    parity.check_checkpoints_against_oracle(prob, dst, pre, st, sc)


@pytest.mark.parametrize("state,rounds", [("bf16", 10), ("i8", 0), ("f8e4m3", 10), ("f32", 0)])
def test_shortest_checkpoint_bit_identical_to_single_call(dev, state, rounds):
    """The shortest positive checkpoint takes exactly the single-call
    arithmetic: its bytes equal rssm_materialize with that prefix."""
    import torch
    import rssm_harness as hx
    spec = ri.with_(CK, state_dtype=state, input_dtype="bf16", philox_rounds=rounds, n_active=5)
    prob = ri.make_problem(spec, 3200)
    rng = np.random.default_rng(3201)
    dst, _ = ri.make_checkpoints(spec, prob.meta, 3202, 3)
    k1 = rng.integers(1, 6, size=spec.B).astype(np.int32)
    pre = np.stack([np.minimum(k1 + rng.integers(1, 4, size=spec.B), spec.W), k1,
                    np.minimum(k1 + rng.integers(0, 4, size=spec.B), spec.W)]).astype(np.int32)
    say("shortest checkpoint vs single call", state, rounds)
    st_multi, sc_multi = run_checkpoints(prob, dst, pre, dev)
    prob1 = copy.deepcopy(prob)
    prob1.meta.prefix[:] = k1
    prob1.meta.dst[:] = dst[1]
    dp = hx.upload(prob1, dev)
    tabs = hx.tables(dp, dev)
    hx.materialize(dp, tabs)
    torch.cuda.synchronize()
    st1 = hx.download(dp.state, prob1.state)
    sc1 = hx.download(dp.scale, prob1.scale) if prob1.scale else None
    n, ns = spec.H * spec.dim * spec.dstate, spec.H * spec.dim
    for l in range(spec.L):
        for i in range(spec.n_active):
            b = int(prob.meta.active[i])
            d = int(dst[1, l, b])
            assert np.array_equal(st_multi[l][d, :n].view(np.uint8), st1[l][d, :n].view(np.uint8)), (l, b)
            if sc1 is not None:
                assert np.array_equal(sc_multi[l][d, :ns].view(np.uint32), sc1[l][d, :ns].view(np.uint32)), (l, b)


def test_one_checkpoint_is_materialize(dev):
    """num_checkpoints = 1 runs the single-checkpoint kernel: same bytes."""
    import torch
    import rssm_harness as hx
    spec = ri.with_(CK, state_dtype="f8e4m3", input_dtype="bf16", philox_rounds=10)
    prob = ri.make_problem(spec, 3300)
    st_a, sc_a = run_checkpoints(prob, prob.meta.dst[None], prob.meta.prefix[None], dev)
    dp = hx.upload(prob, dev)
    tabs = hx.tables(dp, dev)
    hx.materialize(dp, tabs)
    torch.cuda.synchronize()
    st_b = hx.download(dp.state, prob.state)
    sc_b = hx.download(dp.scale, prob.scale)
    for l in range(spec.L):
        assert np.array_equal(st_a[l].view(np.uint8), st_b[l].view(np.uint8))
        assert np.array_equal(sc_a[l].view(np.uint8), sc_b[l].view(np.uint8))


@pytest.mark.parametrize("state,rounds", [("f32", 0), ("bf16", 10), ("i8", 0), ("f8e4m3", 10)])
def test_in_place_flush_single_call(dev, state, rounds):
    """rssm_materialize with every destination equal to its source slot."""
    import torch
    import parity
    import rssm_harness as hx
    spec = ri.with_(CK, state_dtype=state, input_dtype="bf16", philox_rounds=rounds, k0_frac=0.2, pad_frac=0.1)
    prob = ri.make_problem(spec, 3400 + ri.DTYPE_CODE[state])
    m = prob.meta
    m.dst[:] = np.where(m.src == spec.pad_slot_id, spec.pad_slot_id, m.src)
    say("in-place flush", state, rounds)
    expected = __import__("oracle").materialize(prob, want_exact=True)
    dp = hx.upload(prob, dev)
    tabs = hx.tables(dp, dev)
    hx.materialize(dp, tabs)
    torch.cuda.synchronize()
    st = hx.download(dp.state, prob.state)
    sc = hx.download(dp.scale, prob.scale) if prob.scale else None
    parity.check_checkpoints_against_oracle(prob, m.dst[None], m.prefix[None], st, sc, expected=expected)


def test_checkpoints_errors(dev):
    import torch
    import rssm_harness as hx
    import replayssm_persistent_rssm_amd as rp
    spec = ri.with_(CK, state_dtype="bf16")
    prob = ri.make_problem(spec, 3500)
    dp = hx.upload(prob, dev)
    tabs = hx.tables(dp, dev)
    dst = np.stack([prob.meta.dst] * 5)      # five checkpoints: one more than the library takes
    pre = np.stack([prob.meta.prefix] * 5)
    with pytest.raises(rp.RssmError) as e:
        hx.prepared_checkpoints(dp, tabs, i32(dst, dev), i32(pre, dev))()
    assert e.value.status == rp.RSSM_ERR_INVALID_ARGUMENT
    with pytest.raises(ValueError):
        hx.prepared_checkpoints(dp, tabs, i32(dst[0], dev), i32(pre, dev))
    torch.cuda.synchronize()


def test_full_size_flush_and_checkpoint_sampled(dev):
    """large_bf16 at full size in the benchmark's checkpoint configuration: an
    in-place flush of every buffered token plus a checkpoint at half the
    prefix in the request's destination slot; sampled tiles vs the oracle."""
    import torch
    import oracle
    import parity
    import rssm_harness as hx
    spec = ri.CONFIGS["large_bf16"]
    seed = 1002
    say("full size flush + checkpoint, seed", seed)
    dp = ri.make_device_problem(spec, seed, dev, fill_dst=0)
    tabs = hx.tables(dp, dev)
    m = dp.meta
    dst, pre = hx.flush_and_checkpoint_tables(m)
    rng = np.random.default_rng(seed)
    n_tile = spec.dim * spec.dstate
    _, _, d_x, d_B, d_dt = ri.dense_sizes(spec)
    picks = [(0, 0, 0), (spec.B - 1, spec.L - 1, spec.H - 1)]
    picks += [(int(rng.integers(spec.B)), int(rng.integers(spec.L)), int(rng.integers(spec.H))) for _ in range(24)]

    def host(t, sl):
        a = t[sl].cpu()
        if a.dtype == torch.bfloat16:
            a = a.view(torch.int16)
        return a.numpy()
    # the sources are overwritten by the flush: keep the sampled ones first
    src_tiles = {}
    for i, l, h in picks:
        b = int(m.active[i])
        s = int(m.src[l, b])
        src_tiles[(l, b, h)] = host(dp.state[l], (s, slice(h * n_tile, (h + 1) * n_tile))).view(np.uint16).copy()
    call = hx.prepared_checkpoints(dp, tabs, i32(dst, dev), i32(pre, dev))
    call()
    torch.cuda.synchronize()
    for i, l, h in picks:
        b = int(m.active[i])
        s = int(m.src[l, b])
        r0 = int(m.ring_start[b])
        x_slot = host(dp.x[l], (s, slice(0, d_x))).view(np.uint16)
        B_slot = host(dp.Bm[l], (s, slice(0, d_B))).view(np.uint16)
        dt_slot = host(dp.dt[l], (s, slice(0, d_dt)))
        A_h = float(dp.A[l][h].item())
        for c in range(2):
            d, k = int(dst[c, l, b]), int(pre[c, b])
            got = host(dp.state[l], (d, slice(h * n_tile, (h + 1) * n_tile))).view(np.uint16)
            what = f"checkpoint {c} i={i} b={b} l={l} h={h} k={k}"
            if k == 0:
                assert np.array_equal(got, src_tiles[(l, b, h)]), what
                continue
            codes, _, exact, mag = oracle.tile(spec, l, b, h, r0, k, A_h, src_tiles[(l, b, h)], None,
                                               x_slot, B_slot, dt_slot)
            parity.compare_tile(spec.state_dtype, got, codes, exact, mag, None, None, what)
    del dp, tabs, call
    torch.cuda.empty_cache()

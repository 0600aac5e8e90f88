"""Graph capture: a materialize call, a multi-checkpoint call, the decode step
and the gated-delta-rule commit recorded in HIP graphs (torch.cuda.CUDAGraph)
and replayed several times, with the program's own eager work and
synchronisations between replays; every replay must give the bytes of the
eager call.  The library enqueues one kernel per call and no memset, so a
graph holds exactly that launch."""
import sys

import numpy as np
import pytest

import rssm_inputs as ri

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-graph]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import replayssm_persistent_rssm_amd as rp  # noqa: F401
    return torch.device("cuda:0")


def _snapshot(dp):
    import rssm_harness as hx
    st = [a.copy() for a in hx.download(dp.state)]
    sc = [a.copy() for a in hx.download(dp.scale)] if dp.scale else None
    return st, sc


def _same(a, b):
    return all(np.array_equal(x.view(np.uint8), y.view(np.uint8)) for x, y in zip(a, b))


@pytest.mark.parametrize("state,rounds,checkpoints", [("bf16", 0, False), ("f8e4m3", 10, False),
                                                      ("i8", 0, False), ("i8", 0, True)])
def test_graph_replays_match_eager(dev, state, rounds, checkpoints):
    import torch
    import rssm_harness as hx
    spec = ri.Spec("graph", L=3, B=6, H=16, hpg=8, dim=64, dstate=128, R=8, W=8, state_dtype=state,
                   input_dtype="bf16", slots=24, ring_slots=24, slot_mode="perm", philox_rounds=rounds,
                   rand_seed=99, k0_frac=0.2, n_active=5)
    prob = ri.make_problem(spec, 4000 + rounds)
    say(state, rounds, "checkpoints" if checkpoints else "single")
    dp = hx.upload(prob, dev)
    tabs = hx.tables(dp, dev)
    if checkpoints:
        dst, pre = ri.make_checkpoints(spec, prob.meta, 4001, 3)
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)  # noqa: E731
        dst_t, pre_t = i32(dst), i32(pre)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call = hx.prepared_checkpoints(dp, tabs, dst_t, pre_t) if checkpoints else hx.prepared(dp, tabs)
        call()                                     # eager reference on the side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref_st, ref_sc = _snapshot(dp)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gcall = hx.prepared_checkpoints(dp, tabs, dst_t, pre_t) if checkpoints else hx.prepared(dp, tabs)
        gcall()
    for rep in range(3):
        # scribble over every destination slot eagerly, then replay
        for t in dp.state:
            t.view(torch.uint8).fill_(0x5A)
        if dp.scale:
            for t in dp.scale:
                t.view(torch.uint8).fill_(0x5A)
        # restore the sources (inputs) from the host problem
        for t, a in zip(dp.state, prob.state):
            t.copy_(torch.from_numpy(np.ascontiguousarray(a).view(np.uint8)).to(dev).view(t.dtype))
        if dp.scale:
            for t, a in zip(dp.scale, prob.scale):
                t.copy_(torch.from_numpy(np.ascontiguousarray(a)).to(dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        st, sc = _snapshot(dp)
        assert _same(st, ref_st), f"replay {rep}: state differs from the eager call"
        if sc is not None:
            assert _same(sc, ref_sc), f"replay {rep}: scales differ from the eager call"


def _restore_ssu(d, prob):
    """Put the decode step's rings and outputs back to their state before any call."""
    import torch
    fresh = ri.ssu_to_device(prob, d.y.device)
    for name in ("x_ring", "B_ring", "dt_ring"):
        getattr(d, name).copy_(getattr(fresh, name))
    d.y.fill_(float("nan"))


def test_graph_decode_step_replays_match_eager(dev):
    """The checkpointing decode step (ring append + outputs) recorded in a
    graph: each replay, from restored rings, gives the eager call's bytes."""
    import torch
    import rssm_harness as hx
    spec = ri.SSU_CONFIGS["ssu_small"]
    prob = ri.make_ssu_problem(spec, 4200)
    say("decode step")
    d = ri.ssu_to_device(prob, dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        hx.ssu_prepared(d)()                       # eager reference on the side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [a.copy() for a in hx.ssu_download(d)]
    _restore_ssu(d, prob)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gcall = hx.ssu_prepared(d)
        gcall()
    for rep in range(3):
        _restore_ssu(d, prob)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = hx.ssu_download(d)
        for name, a, b in zip(("x ring", "B ring", "dt ring", "y"), got, ref):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"replay {rep}: {name} differs from the eager call"


def test_graph_gdn_commit_replays_match_eager(dev):
    """The gated-delta-rule commit (state updated in place, tracked steps)
    recorded in a graph: each replay, from the restored state, gives the eager
    call's bytes."""
    import torch
    import replayssm_persistent_rssm_amd as rp
    spec = ri.GDN_CONFIGS["gdn_small"]
    prob = ri.make_gdn_problem(spec, 4300)
    say("gdn commit")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    state = t(prob.state)
    args = [state, bf(prob.rawv), bf(prob.rawk), t(prob.g), t(prob.beta), t(prob.state_indices.astype(np.int32)),
            t(prob.accept_lens.astype(np.int32))]
    kw = dict(track_state_indices=t(prob.track_state_indices.astype(np.int32)),
              track_steps=t(prob.track_steps.astype(np.int32)), null_block_id=spec.null_block_id)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rp.GdnCommitCall(*args, **kw)()            # eager reference on the side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = state.cpu().numpy().copy()
    assert not np.array_equal(ref.view(np.uint32), prob.state.view(np.uint32)), "the eager call wrote nothing"
    state.copy_(t(prob.state))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gcall = rp.GdnCommitCall(*args, **kw)
        gcall()
    for rep in range(3):
        state.copy_(t(prob.state))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(state.cpu().numpy().view(np.uint32), ref.view(np.uint32)), \
            f"replay {rep}: state differs from the eager call"

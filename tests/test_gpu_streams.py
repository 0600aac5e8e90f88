"""Calls on different streams and from different host threads are
independent.  The library keeps no state between calls beyond per-thread
caches and no device memory of its own, so calls enqueued on two streams (and
free to run at the same time) give what each gives alone: checked against the
oracle for two different instances side by side, for one pool whose active
requests are split over two streams, and for three host threads calling at
once."""
import sys

import numpy as np
import pytest

import rssm_inputs as ri

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-streams]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import replayssm_persistent_rssm_amd as rp  # noqa: F401  (fails loudly if the library is missing)
    return torch.device("cuda:0")


def _spec(state, inp, rounds, B=6):
    return ri.Spec("streams", L=3, B=B, H=16, hpg=8, dim=64, dstate=128, R=8, W=8, state_dtype=state,
                   input_dtype=inp, slots=2 * B, ring_slots=2 * B, slot_mode="split", philox_rounds=rounds,
                   rand_seed=321, k0_frac=0.2)


def _result(dp, prob):
    import rssm_harness as hx
    st = hx.download(dp.state, prob.state)
    sc = hx.download(dp.scale, prob.scale) if prob.scale else None
    return st, sc


def test_two_instances_on_two_streams(dev):
    """bf16 on the vector-ALU fold and e4m3 + Philox on the matrix-core fold
    (eight times the resident grid), each on its own stream and pools, each
    enqueued three times without synchronisation in between."""
    import torch
    import parity
    import rssm_harness as hx
    probs = [ri.make_problem(_spec("bf16", "bf16", 0), 4400), ri.make_problem(_spec("f8e4m3", "bf16", 10), 4401)]
    dps = [hx.upload(p, dev) for p in probs]
    tabs = [hx.tables(dp, dev) for dp in dps]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    calls = [hx.prepared(dp, tb, stream=s) for dp, tb, s in zip(dps, tabs, streams)]
    say("two instances, two streams")
    for _ in range(3):          # destinations and sources are disjoint: every call writes the same bytes
        for c in calls:
            c()
    torch.cuda.synchronize()
    for p, dp in zip(probs, dps):
        st, sc = _result(dp, p)
        parity.check_against_oracle(p, st, sc)


def test_one_pool_split_over_two_streams(dev):
    """The active requests of one batch split over two streams writing the
    same pools (disjoint destination slots): the pools end as after one call
    with every request."""
    import torch
    import parity
    import rssm_harness as hx
    for state, inp, rounds in (("bf16", "bf16", 0), ("i8", "f16", 0)):
        prob = ri.make_problem(_spec(state, inp, rounds, B=8), 4410)
        act = [int(v) for v in prob.meta.active if v >= 0]
        assert len(act) == prob.spec.B
        dp = hx.upload(prob, dev)
        halves = []
        for part in (act[0::2], act[1::2]):
            a = np.full(prob.spec.B, -1, np.int32)
            a[:len(part)] = part
            halves.append(hx.tables(dp, dev, active=a))
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        say("one pool, split active list", state)
        calls = [hx.prepared(dp, tb, stream=s) for tb, s in zip(halves, streams)]
        for c in calls:
            c()
        torch.cuda.synchronize()
        st, sc = _result(dp, prob)
        parity.check_against_oracle(prob, st, sc)


def test_host_threads_share_the_library(dev):
    """Three host threads use the library at once (a ctypes call releases the
    interpreter lock, so they overlap inside it).  Two alternate between two
    instances each, on a stream of their own, so the per-thread launch cache
    changes descriptor on every call; the third repeatedly makes calls that
    fail host validation, whose error text must stay its own.  Every pool
    must then hold the oracle's result."""
    import threading
    import torch
    import parity
    import rssm_harness as hx
    import replayssm_persistent_rssm_amd as rp
    kinds = [("bf16", "bf16", 0), ("i8", "f16", 0), ("f16", "f32", 7), ("f8e4m3", "bf16", 10)]
    probs = [ri.make_problem(_spec(*k), 4500 + j) for j, k in enumerate(kinds)]
    dps = [hx.upload(p, dev) for p in probs]
    tabs = [hx.tables(dp, dev) for dp in dps]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    # thread t owns problems 2t and 2t+1 and stream t
    calls = [[hx.prepared(dps[2 * t + q], tabs[2 * t + q], stream=streams[t]) for q in range(2)] for t in range(2)]
    errors = []
    bad_texts = []

    def worker(t):
        try:
            for n in range(200):
                calls[t][n % 2]()
        except Exception as e:  # noqa: BLE001  (reported below)
            errors.append(repr(e))

    def failing():
        for n in range(200):
            try:
                rp.rssm_materialize_launch_config(num_layers=0, batch=1, num_heads=1, heads_per_group=1, dim=64,
                                                  dstate=128, max_window=8, ring_buffer_len=8, state_dtype="bf16",
                                                  input_dtype="bf16")
                bad_texts.append("no error")
            except rp.RssmError:
                text = rp.rssm_last_error()
                if "num_layers" not in text:
                    bad_texts.append(text)

    say("three host threads, 200 calls each")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)] + [threading.Thread(target=failing)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a host thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    assert not bad_texts, bad_texts[:3]
    for p, dp in zip(probs, dps):
        parity.check_against_oracle(p, *_result(dp, p))

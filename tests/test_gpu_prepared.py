"""Prepared calls (MaterializeCall, GdnCommitCall, SsuDecodeCall) keep their
tensors allocated.

Their descriptor tables hold bare device addresses, so a prepared call built
from tensors that its caller then drops would read freed memory at the next
call.  Each test here builds a call from tables that nothing else
references, drops them, and checks through weak references that the call
still holds every one of them BEFORE it launches anything; the materialize
case then runs the call (twice, the second time with a dropped active list)
and compares with the oracle.
"""
import gc
import sys
import weakref

import numpy as np
import pytest

import rssm_inputs as ri

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-prepared]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import replayssm_persistent_rssm_amd as rp  # noqa: F401  (fails loudly if the library is missing)
    return torch.device("cuda:0")


def _tensors(obj):
    import torch
    return [v for v in vars(obj).values() if isinstance(v, torch.Tensor)]


def _all_alive(refs):
    gc.collect()
    return all(r() is not None for r in refs)


def test_materialize_call_holds_its_tables(dev):
    import torch
    import parity
    import rssm_harness as hx
    prob = ri.make_problem(ri.CONFIGS["mid_bf16"], 310)
    dp = hx.upload(prob, dev)
    tabs = hx.tables(dp, dev)
    refs = [weakref.ref(t) for t in _tensors(tabs)]
    assert len(refs) >= 14
    call = hx.prepared(dp, tabs)
    del tabs
    assert _all_alive(refs), "a prepared call let its tables be freed"
    say("mid_bf16: prepared call from dropped tables, launching")
    call()
    torch.cuda.synchronize()
    parity.check_against_oracle(prob, hx.download(dp.state, prob.state), None)

    # a dropped active list passed to a call is held as well (same requests,
    # so the second call writes the same values again)
    act = torch.from_numpy(np.ascontiguousarray(prob.meta.active, np.int32)).to(dev)
    wa = weakref.ref(act)
    call(act)
    del act
    assert _all_alive([wa]), "a prepared call let its active list be freed"
    call()
    torch.cuda.synchronize()
    parity.check_against_oracle(prob, hx.download(dp.state, prob.state), None)


def test_gdn_and_ssu_calls_hold_their_tensors(dev):
    import torch
    import replayssm_persistent_rssm_amd as rp
    import rssm_harness as hx
    gp = ri.make_gdn_problem(ri.GDN_CONFIGS["gdn_small"], 311)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    args = [t(gp.state), bf(gp.rawv), bf(gp.rawk), t(gp.g), t(gp.beta), t(gp.state_indices.astype(np.int32)),
            t(gp.accept_lens.astype(np.int32))]
    refs = [weakref.ref(a) for a in args]
    call = rp.GdnCommitCall(*args, null_block_id=gp.spec.null_block_id)
    del args
    assert _all_alive(refs), "GdnCommitCall let its tensors be freed"

    sp = ri.make_ssu_problem(ri.SSU_CONFIGS["ssu_small"], 312)
    d = ri.ssu_to_device(sp, dev)
    slots = d.slots.clone()   # referenced by nothing but the call
    ws = weakref.ref(slots)
    args, kw = hx._ssu_args(d, 0)
    args = list(args)
    args[10] = slots
    scall = rp.SsuDecodeCall(*args, **kw)
    del slots, args
    assert _all_alive([ws]), "SsuDecodeCall let its tensors be freed"
    del call, scall

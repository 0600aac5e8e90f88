"""Seeded random workload shapes against the oracle: every compiled state x
input dtype pair, both tile shapes, windows of 8 and 16, ring lengths below
and above the window, head groupings, pad pairs, slot-stride gaps, slot
layouts, partial active lists and stochastic rounding, drawn together so that
their combinations are exercised, not only each on its own.  The draws are
fixed by the seed; every case is small enough for the oracle."""
import sys

import numpy as np
import pytest

import rssm_inputs as ri

pytestmark = pytest.mark.gpu

STATES = ["f32", "bf16", "f16", "i8", "f8e4m3"]
INPUTS = ["f32", "bf16", "f16"]


def say(*a):
    print("[gpu-random]", *a, flush=True)
    sys.stdout.flush()


def draw(i: int) -> ri.Spec:
    rng = np.random.default_rng(9100 + i)
    state = STATES[i % len(STATES)]
    inp = INPUTS[int(rng.integers(len(INPUTS)))]
    big = state in ("i8", "f8e4m3") or rng.random() < 0.4
    dim, dstate = (64, 128) if big else (16, 16)
    W = int(rng.choice([8, 16]))
    R = int(rng.integers(1, 2 * W + 3))
    G = int(rng.integers(1, 4))
    hpg = int(rng.integers(1, 5))
    H = G * hpg if big else min(G * hpg * int(rng.integers(1, 4)), 24)
    H -= H % hpg
    H = max(H, hpg)
    L = int(rng.integers(1, 5 if big else 9))
    B = int(rng.integers(1, 7 if big else 13))
    rounds = 0 if state == "f32" or rng.random() < 0.5 else int(rng.choice([1, 7, 10]))
    return ri.Spec(f"random{i}", L=L, B=B, H=H, hpg=hpg, dim=dim, dstate=dstate, R=R, W=W, state_dtype=state,
                   input_dtype=inp, n_active=int(rng.integers(1, B + 1)), k_lo=0, k_hi=W,
                   k0_frac=float(rng.choice([0.0, 0.25])), slot_mode=str(rng.choice(["split", "perm"])),
                   stride_pad=str(rng.choice(["none", "per_layer"])), pad_frac=float(rng.choice([0.0, 0.3])),
                   philox_rounds=rounds, rand_seed=int(rng.integers(1, 2**62)) if rounds else None)


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import replayssm_persistent_rssm_amd as rp  # noqa: F401  (fails loudly if the library is missing)
    return torch.device("cuda:0")


@pytest.mark.parametrize("i", range(64))
def test_random_spec_matches_oracle(dev, i):
    import test_gpu_parity as tp
    spec = draw(i)
    prob = ri.make_problem(spec, 9200 + i)
    say(i, f"L={spec.L} B={spec.B} active={spec.n_active} H={spec.H} hpg={spec.hpg} {spec.dim}x{spec.dstate} "
           f"{spec.state_dtype}/{spec.input_dtype} W={spec.W} R={spec.R} rounds={spec.philox_rounds} "
           f"{spec.slot_mode} {spec.stride_pad} pads={spec.pad_frac}")
    tp.check(prob, dev)

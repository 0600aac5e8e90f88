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


@pytest.mark.parametrize("i", range(256))
def test_random_spec_matches_oracle(dev, i):
    import test_gpu_parity as tp
    spec = draw(i)
    prob = ri.make_problem(spec, 9200 + i)
    say(i, f"L={spec.L} B={spec.B} active={spec.n_active} H={spec.H} hpg={spec.hpg} {spec.dim}x{spec.dstate} "
           f"{spec.state_dtype}/{spec.input_dtype} W={spec.W} R={spec.R} rounds={spec.philox_rounds} "
           f"{spec.slot_mode} {spec.stride_pad} pads={spec.pad_frac}")
    tp.check(prob, dev)


def draw_checkpoints(i: int):
    """A random multi-checkpoint case (64 x 128 tiles, the compiled shape)."""
    rng = np.random.default_rng(9300 + i)
    state = STATES[i % len(STATES)]
    inp = INPUTS[int(rng.integers(len(INPUTS)))]
    W = int(rng.choice([8, 16]))
    hpg = int(rng.integers(1, 4))
    H = hpg * int(rng.integers(1, 3))
    L = int(rng.integers(1, 4))
    B = int(rng.integers(1, 6))
    n_ck = int(rng.integers(1, 5))
    rounds = 0 if state == "f32" or rng.random() < 0.5 else int(rng.choice([1, 10]))
    spec = ri.Spec(f"ckrandom{i}", L=L, B=B, H=H, hpg=hpg, dim=64, dstate=128, R=int(rng.integers(1, 2 * W + 3)),
                   W=W, state_dtype=state, input_dtype=inp, n_active=int(rng.integers(1, B + 1)), k_lo=0, k_hi=W,
                   slots=(n_ck + 2) * B, ring_slots=(n_ck + 2) * B, slot_mode="perm",
                   stride_pad=str(rng.choice(["none", "per_layer"])), pad_frac=float(rng.choice([0.0, 0.3])),
                   philox_rounds=rounds, rand_seed=int(rng.integers(1, 2**62)) if rounds else None)
    opts = dict(in_place=bool(rng.random() < 0.5), k0_frac=float(rng.choice([0.0, 0.3])),
                pad_frac=float(rng.choice([0.0, 0.3])), dup_frac=float(rng.choice([0.0, 0.3])))
    return spec, n_ck, opts


@pytest.mark.parametrize("i", range(96))
def test_random_checkpoint_spec_matches_oracle(dev, i):
    import parity
    import test_gpu_checkpoints as tc
    spec, n_ck, opts = draw_checkpoints(i)
    prob = ri.make_problem(spec, 9400 + i)
    dst, pre = ri.make_checkpoints(spec, prob.meta, 9500 + i, n_ck, **opts)
    say("checkpoints", i, f"L={spec.L} B={spec.B} active={spec.n_active} H={spec.H} hpg={spec.hpg} "
                          f"{spec.state_dtype}/{spec.input_dtype} W={spec.W} R={spec.R} n_ck={n_ck} {opts} "
                          f"rounds={spec.philox_rounds}")
    st, sc = tc.run_checkpoints(prob, dst, pre, dev)
    parity.check_checkpoints_against_oracle(prob, dst, pre, st, sc)


def draw_gdn(i: int) -> "ri.GdnSpec":
    """A random gated-delta-rule commit (128 x 128 fp32 states)."""
    rng = np.random.default_rng(9600 + i)
    H = int(rng.integers(1, 3))
    B = int(rng.integers(1, 7))
    return ri.GdnSpec(f"gdnrandom{i}", L=int(rng.integers(1, 3)), B=B, HV=H * int(rng.integers(1, 3)), H=H,
                      T=int(rng.integers(1, 17)), slots=3 * B + 2, use_l2norm=bool(rng.random() < 0.75),
                      null_block_id=int(rng.choice([-1, 0])), null_frac=float(rng.choice([0.0, 0.3])),
                      track=bool(rng.random() < 0.6), zero_frac=float(rng.choice([0.0, 0.2])))


@pytest.mark.parametrize("i", range(64))
def test_random_gdn_spec_matches_oracle(dev, i):
    import test_gpu_gdn as tg
    spec = draw_gdn(i)
    prob = ri.make_gdn_problem(spec, 9700 + i)
    if not spec.use_l2norm:
        # unnormalised keys scaled to |k|^2 < 2, so the update stays non-expanding
        k = (prob.rawk.astype(np.uint32) << 16).view(np.float32) * np.float32(1.0 / 16)
        prob.rawk = ri._bf16_codes(k)
    say("gdn", i, spec)
    tg.check(prob, tg.run(prob, dev), f"gdn random {i}")


def draw_ssu(i: int) -> "ri.SsuSpec":
    """A random decode step (64 x 128 checkpoints, the compiled shape)."""
    rng = np.random.default_rng(9800 + i)
    hpg = int(rng.integers(1, 5))
    T = int(rng.integers(1, 9))
    R = int(rng.integers(T, 17))
    softplus = bool(rng.random() < 0.7)
    # the drawn bias is softplus^-1 of a small step (negative): without the
    # softplus it would make dt negative, which is no timestep, and |dt A|
    # far beyond the range the output tolerance is derived for
    bias = softplus and bool(rng.random() < 0.7)
    return ri.SsuSpec(f"ssurandom{i}", B=int(rng.integers(1, 7)), H=hpg * int(rng.integers(1, 3)), hpg=hpg,
                      dim=64, dstate=128, R=R, T=T, state_dtype=STATES[i % 3], input_dtype=INPUTS[int(rng.integers(3))],
                      has_z=bool(rng.random() < 0.7), has_D=bool(rng.random() < 0.7),
                      has_bias=bias, dt_softplus=softplus, pad_frac=float(rng.choice([0.0, 0.3])))


@pytest.mark.parametrize("i", range(64))
def test_random_decode_spec_matches_oracle(dev, i):
    import test_gpu_ssu as ts
    spec = draw_ssu(i)
    prob = ri.make_ssu_problem(spec, 9900 + i)
    say("decode", i, spec)
    ts.check(prob, ts.run(prob, dev), f"decode random {i}")

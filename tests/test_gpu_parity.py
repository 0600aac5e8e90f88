"""GPU parity: librssm_materialize (through its C ABI) against the CPU oracle.

Every case draws seeded inputs from rssm_inputs, runs the oracle on the host
and the HIP path on the device, and compares element by element with the
tolerances of tests/parity.py.  Full-size workloads are checked on sampled
tiles that the oracle computes one by one, in the launch configuration the
benchmark times.
"""
import hashlib
import sys

import numpy as np
import pytest

import rssm_inputs as ri

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import replayssm_persistent_rssm_amd as rp  # noqa: F401  (fails loudly if the library is missing)
    return torch.device("cuda:0")


def run_gpu(prob, dev, max_workgroups=0, active=None):
    import torch
    import rssm_harness as hx
    dp = hx.upload(prob, dev)
    tabs = hx.tables(dp, dev)
    act = None
    if active is not None:
        act = torch.from_numpy(np.ascontiguousarray(active, np.int32)).to(dev)
    hx.materialize(dp, tabs, max_workgroups=max_workgroups, active=act)
    torch.cuda.synchronize()
    st = hx.download(dp.state, prob.state)
    sc = hx.download(dp.scale, prob.scale) if prob.scale else None
    ring = [hx.download(dp.x, prob.x), hx.download(dp.Bm, prob.Bm), hx.download(dp.dt, prob.dt),
            hx.download(dp.A, prob.A)]
    return st, sc, ring


def check(prob, dev, expected=None, **kw):
    import parity
    st, sc, ring = run_gpu(prob, dev, **kw)
    for got, want in zip(ring, [prob.x, prob.Bm, prob.dt, prob.A]):
        for g, w in zip(got, want):
            assert np.array_equal(g.view(np.uint8), w.view(np.uint8)), "ring or A changed"
    parity.check_against_oracle(prob, st, sc, expected)
    return st, sc


# --------------------------------------------------------------------------
# The workloads' own shapes (small ones whole; large ones scaled down here,
# sampled at full size below)
# --------------------------------------------------------------------------
def test_tiny_f32_workload(dev):
    spec = ri.CONFIGS["tiny_f32"]
    say("tiny_f32 seed 1000", spec)
    check(ri.make_problem(spec, 1000), dev)


def test_mid_bf16_workload(dev):
    spec = ri.CONFIGS["mid_bf16"]
    say("mid_bf16 seed 1001 (distinct strides per layer)")
    check(ri.make_problem(spec, 1001), dev)


SCALED = {
    "large_bf16": dict(L=3, B=8, H=64, n_active=5, slots=16, ring_slots=8),
    "large_i8": dict(L=2, B=8, H=64, n_active=6, slots=16, ring_slots=8),
    "large_f8sr": dict(L=2, B=8, H=32, n_active=5, slots=16, ring_slots=8),
}


@pytest.mark.parametrize("name", list(SCALED))
def test_large_workloads_scaled(dev, name):
    spec = ri.scaled(ri.CONFIGS[name], name + "_scaled", **SCALED[name])
    say(name, "scaled", SCALED[name])
    check(ri.make_problem(spec, 1002 + list(SCALED).index(name)), dev)


# --------------------------------------------------------------------------
# dtype matrix on the 64x128 tile, plus the 16x16 tile
# --------------------------------------------------------------------------
MATRIX = ri.Spec("matrix", L=2, B=3, H=8, hpg=4, dim=64, dstate=128, R=8, W=8, k_lo=0, k_hi=8,
                 slots=6, ring_slots=6, slot_mode="perm", stride_pad="per_layer", rand_seed=77)


@pytest.mark.parametrize("state", ["f32", "bf16", "f16", "i8", "f8e4m3"])
@pytest.mark.parametrize("inp", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("rounds", [0, 10])
def test_dtype_matrix(dev, state, inp, rounds):
    if state == "f32" and rounds:
        pytest.skip("fp32 state is never rounded")
    spec = ri.with_(MATRIX, state_dtype=state, input_dtype=inp, philox_rounds=rounds)
    say("matrix", state, inp, rounds)
    check(ri.make_problem(spec, 2000 + ri.DTYPE_CODE[state] * 10 + ri.DTYPE_CODE[inp]), dev)


# More than 256 requests: the active-list scan pages through the list 256
# entries at a time, and the kernel reads request indices past 255 from memory.
BIG_BATCH = ri.Spec("big_batch", L=2, B=600, H=2, hpg=1, dim=64, dstate=128, R=8, W=8, k_lo=0, k_hi=8,
                    slots=1300, slot_mode="perm", pad_frac=0.1, rand_seed=91)


@pytest.mark.parametrize("state,inp,rounds,n_active", [
    ("bf16", "bf16", 0, 256), ("bf16", "bf16", 0, 257), ("bf16", "bf16", 0, 600),
    ("i8", "f16", 0, 450), ("f8e4m3", "bf16", 10, 450)])
def test_batch_over_256(dev, state, inp, rounds, n_active):
    """600 requests (450 listed, or the list ending at 256 / 257 / not at all),
    a tenth of the (layer, request) pairs padded; the default grid, and 8
    workgroups, where every wavefront deals many chunks and filters their
    liveness in batches.  One oracle result serves both launches."""
    import oracle
    import parity
    spec = ri.with_(BIG_BATCH, state_dtype=state, input_dtype=inp, philox_rounds=rounds, n_active=n_active)
    prob = ri.make_problem(spec, 2400 + n_active)
    expected = oracle.materialize(prob, want_exact=True)
    for mw in (0, 8):
        say("big batch", state, inp, rounds, n_active, "max_workgroups", mw)
        st, sc, _ = run_gpu(prob, dev, max_workgroups=mw)
        parity.check_against_oracle(prob, st, sc, expected=expected)


@pytest.mark.parametrize("state", ["f32", "bf16", "f16"])
def test_small_tile_16x16(dev, state):
    spec = ri.with_(ri.CONFIGS["tiny_f32"], name="t16", L=2, B=5, H=6, hpg=3, state_dtype=state,
                    input_dtype="bf16", ring_start=None, prefix=None, k_lo=0, k_hi=8, slots=10, ring_slots=10,
                    slot_mode="perm", src_fixed=None, dst_fixed=None, stride_pad="per_layer",
                    active_order="random", philox_rounds=7 if state != "f32" else 0, rand_seed=5)
    say("16x16", state)
    check(ri.make_problem(spec, 2100 + ri.DTYPE_CODE[state]), dev)


def test_window_16_and_short_ring(dev):
    """max_window 16 (the wide-register instance) with a ring shorter than the
    window: entries wrap more than once."""
    spec = ri.with_(MATRIX, W=16, R=5, k_lo=9, k_hi=16, state_dtype="bf16", input_dtype="bf16")
    say("W=16 R=5")
    check(ri.make_problem(spec, 2200), dev)


@pytest.mark.parametrize("state,inp,rounds", [
    ("f32", "bf16", 0), ("f32", "f32", 0), ("bf16", "bf16", 10), ("bf16", "f32", 0), ("f16", "f16", 0),
    ("i8", "f16", 0), ("i8", "bf16", 10), ("f8e4m3", "bf16", 10), ("f8e4m3", "f32", 0)])
def test_window_16_dtypes(dev, state, inp, rounds):
    """16-token windows for every state dtype (B rows of tokens 4..15 come from
    the wavefront's LDS): prefixes U[0, 16], 4 B groups per (request, layer) so
    each group rewrites those rows, and a ring longer than the window."""
    spec = ri.with_(MATRIX, W=16, R=21, k_lo=0, k_hi=16, H=8, hpg=2, B=4, slots=8, ring_slots=8,
                    state_dtype=state, input_dtype=inp, philox_rounds=rounds)
    say("window 16", state, inp, rounds)
    check(ri.make_problem(spec, 2600 + 10 * ri.DTYPE_CODE[state] + ri.DTYPE_CODE[inp]), dev)


# --------------------------------------------------------------------------
# Edge cases
# --------------------------------------------------------------------------
def test_no_active_request(dev):
    prob = ri.make_problem(ri.with_(MATRIX, n_active=0), 2300)
    say("n_active=0")
    check(prob, dev)


def test_all_pad_and_nondefault_pad(dev):
    spec = ri.with_(MATRIX, pad_slot_id=3, slot_mode="fixed", src_fixed=[0, 3, 1], dst_fixed=[4, 5, 3],
                    stride_pad="none")
    prob = ri.make_problem(spec, 2301)
    say("pad_slot_id=3, slot 0 valid")
    check(prob, dev)
    prob2 = ri.make_problem(ri.with_(MATRIX, pad_frac=1.0), 2302)
    say("every pair padded")
    check(prob2, dev)


@pytest.mark.parametrize("H,hpg", [(8, 4), (4, 2), (24, 8)])
@pytest.mark.parametrize("pad_frac", [0.5, 0.97])
def test_mixed_pads_many_chunks_per_wave(dev, H, hpg, pad_frac):
    """Padded (layer, request) pairs mixed with live ones while each wavefront
    deals many chunks: grids of 1-7 workgroups give up to 100+ chunks per
    wavefront, so the kernel tests chunk liveness in several batches of 64
    and skips dead ones.  H = 4 and 24 make chunks of 16 heads straddle
    (request, layer) pairs; pad_frac 0.97 leaves whole batches dead."""
    spec = ri.with_(MATRIX, L=8, B=40, H=H, hpg=hpg, dim=16, dstate=16, slots=80, ring_slots=80,
                    n_active=36, pad_frac=pad_frac, stride_pad="per_layer")
    prob = ri.make_problem(spec, 2310 + H + int(pad_frac * 100))
    for mw in (1, 3, 7, 0):
        say("mixed pads H", H, "pad_frac", pad_frac, "grid", mw)
        check(prob, dev, max_workgroups=mw)


def test_all_listed_all_pad_many_chunks(dev):
    """Every listed request padded in every layer, with enough items that each
    wavefront of the default grid deals several chunks: nothing is written."""
    spec = ri.with_(MATRIX, L=48, B=48, H=32, hpg=8, dim=16, dstate=16, slots=96, ring_slots=96,
                    n_active=48, pad_frac=1.0, stride_pad="none")
    prob = ri.make_problem(spec, 2320)
    for mw in (0, 2):
        say("all listed, all padded; grid", mw)
        check(prob, dev, max_workgroups=mw)


@pytest.mark.parametrize("state,inp,dim,dstate,rounds", [("bf16", "bf16", 16, 16, 0), ("f32", "f16", 16, 16, 0),
                                                         ("i8", "f16", 64, 128, 0), ("f8e4m3", "bf16", 64, 128, 10)])
def test_more_layers_than_a_wavefront(dev, state, inp, dim, dstate, rounds):
    """80 layers (more than one wavefront's 64 lanes) with padded pairs mixed
    in: every per-layer table is read at indices past 63, chunks straddle
    (request, layer) pairs (H = 6), and the one-byte cases run the
    matrix-core fold."""
    spec = ri.with_(MATRIX, L=80, B=3, H=6 if dim == 16 else 2, hpg=3 if dim == 16 else 1, dim=dim, dstate=dstate,
                    state_dtype=state, input_dtype=inp, philox_rounds=rounds, slots=6, ring_slots=6,
                    pad_frac=0.2, stride_pad="per_layer")
    prob = ri.make_problem(spec, 2330 + dim + rounds)
    expected = oracle_result(prob)
    for mw in (0, 5):
        say("80 layers", state, inp, f"{dim}x{dstate}", "rounds", rounds, "grid", mw)
        check(prob, dev, expected, max_workgroups=mw)


@pytest.mark.parametrize("state,inp", [("bf16", "bf16"), ("i8", "f16")])
def test_out_of_range_metadata_guards(dev, state, inp):
    """Device metadata outside its documented range is undefined on the
    pages; the kernel guards against faults instead: k is clamped to
    [0, max_window], ring_start is taken modulo R, a negative source or
    destination slot skips its (layer, request), and an active entry outside
    [0, B) ends the list.  The result must equal the oracle's on metadata
    sanitised that way (the oracle itself rejects such values)."""
    import copy
    import parity
    spec = ri.with_(MATRIX, B=6, slots=12, ring_slots=12, state_dtype=state, input_dtype=inp)
    bad = ri.make_problem(spec, 2340)
    m, W, R, pad = bad.meta, spec.W, spec.R, spec.pad_slot_id
    act = [int(v) for v in m.active[:5]]
    assert len(set(act)) == 5 and min(act) >= 0
    m.prefix[act[0]] = W + 9                  # clamped to W
    m.prefix[act[1]] = -4                     # clamped to 0: a copy
    m.ring_start[act[2]] = -11                # taken modulo R
    m.ring_start[act[3]] = 3 * R + 5
    m.src[0, act[0]] = -5                     # negative slots (not the pad id): skipped
    m.dst[1, act[1]] = -9
    m.active[4] = spec.B + 3                  # out of range: ends the list
    m.active[5] = act[4]                      # after the end: ignored
    sane = copy.copy(bad)
    sane.meta = copy.deepcopy(m)
    sm = sane.meta
    sm.active[4:] = -1
    sm.prefix[:] = np.clip(sm.prefix, 0, W)
    sm.ring_start[:] = np.mod(sm.ring_start, R)
    neg = (sm.src < 0) & (sm.src != pad) | (sm.dst < 0) & (sm.dst != pad)
    sm.src[neg] = pad
    sm.dst[neg] = pad
    say("out-of-range metadata", state, inp)
    st, sc, ring = run_gpu(bad, dev)
    for got, want in zip(ring, [bad.x, bad.Bm, bad.dt, bad.A]):
        for g, w in zip(got, want):
            assert np.array_equal(g.view(np.uint8), w.view(np.uint8)), "ring or A changed"
    parity.check_against_oracle(sane, st, sc)


def test_entries_after_first_terminator_ignored(dev):
    prob = ri.make_problem(ri.with_(MATRIX, n_active=3), 2303)
    prob.meta.active[1] = -1                  # only the first request counts
    say("garbage after -1")
    check(prob, dev)


def test_ragged_batch_across_wave_boundaries(dev):
    """B = 70 (spans two 64-entry ballots) with 69 active, tiny tiles: the
    work does not divide the grid."""
    spec = ri.with_(ri.CONFIGS["tiny_f32"], name="ragged", L=2, B=70, H=2, hpg=1, ring_start=None,
                    prefix=None, k_lo=0, k_hi=8, slots=140, ring_slots=140, slot_mode="perm",
                    src_fixed=None, dst_fixed=None, n_active=69, active_order="random")
    say("ragged B=70 n=69")
    check(ri.make_problem(spec, 2304), dev)


def _digest(arrs):
    h = hashlib.sha256()
    for a in arrs:
        h.update(np.ascontiguousarray(a).view(np.uint8).tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("state,rounds", [("bf16", 0), ("f8e4m3", 10), ("i8", 10)])
def test_grid_and_order_invariance(dev, state, rounds):
    """Results do not depend on the persistent grid size or on the order of
    the active prefix (Philox keys use the physical request index)."""
    spec = ri.with_(MATRIX, state_dtype=state, input_dtype="bf16", philox_rounds=rounds, B=5, slots=10,
                    ring_slots=10, n_active=4)
    prob = ri.make_problem(spec, 2400)
    digests = set()
    for mw in (0, 1, 2, 7, 1000):
        say("grid", mw, state)
        st, sc, _ = run_gpu(prob, dev, max_workgroups=mw)
        digests.add(_digest(st + (sc or [])))
    act = prob.meta.active.copy()
    act[:4] = act[:4][::-1]
    st, sc, _ = run_gpu(prob, dev, active=act)
    digests.add(_digest(st + (sc or [])))
    assert len(digests) == 1


# --------------------------------------------------------------------------
# Rounding: bit-exact against the oracle when pre-rounding values agree
# --------------------------------------------------------------------------
def _exact_arithmetic(prob):
    """A = 0, dt = 2^-4, x small integers, B integers / 16, state a multiple
    of 2^-8 (one-byte: power-of-two row scales): every fp32 value on both
    sides is exact, so codes must agree bit for bit."""
    rng = np.random.default_rng(99)
    s = prob.spec
    for l in range(s.L):
        prob.A[l][:] = 0.0
        prob.dt[l][:] = 2.0 ** -4
        xv = rng.integers(-3, 4, size=prob.x[l].shape).astype(np.float32)
        bv = (rng.integers(-8, 9, size=prob.Bm[l].shape) / 16.0).astype(np.float32)
        prob.x[l][:] = ri._to_storage(xv, s.input_dtype)
        prob.Bm[l][:] = ri._to_storage(bv, s.input_dtype)
        if ri.one_byte(s.state_dtype):
            prob.scale[l][:] = 2.0 ** -5
            # every finite code appears (e4m3: all but the two NaN codes)
            n = prob.state[l].size
            if s.state_dtype == "f8e4m3":
                finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
            else:
                finite = np.arange(-127, 128).astype(np.int8)
            prob.state[l].reshape(-1)[:] = np.resize(rng.permutation(finite), n)
        else:
            sv = (rng.integers(-1024, 1025, size=prob.state[l].shape) / 256.0).astype(np.float32)
            prob.state[l][:] = ri._to_storage(sv, s.state_dtype)
    return prob


@pytest.mark.parametrize("state", ["bf16", "f16", "i8", "f8e4m3"])
@pytest.mark.parametrize("rounds", [0, 10])
@pytest.mark.parametrize("window,inp", [(8, "bf16"), (16, "bf16"), (8, "f16")])
def test_rounding_bit_exact_on_exact_inputs(dev, state, rounds, window, inp):
    """Every code bit-exact where both sides hold the same fp32 values; window
    16 takes the instances that keep B rows 4..15 in LDS, fp16 inputs with
    int8 state the instance that multiplies packed fp16 B rows."""
    import oracle
    spec = ri.with_(MATRIX, state_dtype=state, input_dtype=inp, philox_rounds=rounds, rand_seed=1234,
                    W=window, k_hi=window, R=window + 3, hpg=2 if window > 8 else MATRIX.hpg)
    prob = _exact_arithmetic(ri.make_problem(spec, 2500 + window))
    say("bit-exact rounding", state, rounds, "window", window, "input", inp)
    st, sc, _ = run_gpu(prob, dev)
    st_o, sc_o, ex, _ = oracle.materialize(prob, want_exact=True)
    for l in range(spec.L):
        g, o = st[l].view(np.uint8), st_o[l].view(np.uint8)
        if not np.array_equal(g, o):
            eb = ri.ELEM_BYTES[state]
            bad = np.argwhere(g != o)[:8]
            lines = []
            for slot, byte in bad:
                e = byte // eb
                lines.append(f"slot {slot} elem {e} (head {e // (spec.dim * spec.dstate)}): gpu "
                             f"{g[slot, e * eb:(e + 1) * eb].tobytes().hex()} oracle "
                             f"{o[slot, e * eb:(e + 1) * eb].tobytes().hex()} exact {ex[l][slot, e]!r}")
            pytest.fail(f"layer {l}: {int((g != o).sum())} bytes differ; first: " + "; ".join(lines))
        if sc is not None:
            assert np.array_equal(sc[l].view(np.uint32), sc_o[l].view(np.uint32)), f"layer {l} scales differ"


@pytest.mark.parametrize("state,rounds", [("i8", 0), ("i8", 10), ("f8e4m3", 0), ("f8e4m3", 10)])
@pytest.mark.parametrize("window", [8, 16])
def test_one_byte_special_rows(dev, state, rounds, window):
    """Rows the one-byte encode treats specially, through the whole kernel (the
    matrix-core fold's row-block encode), in every written source slot: an
    all-zero row (zero codes and x entries: scale 0, zero codes), a row whose
    huge source scale overflows to infinity (scale 0, zero codes) and, for
    e4m3, a NaN source code inside an otherwise normal row (the NaN code of
    either sign at that element, the row's other codes and scale unchanged by
    it)."""
    spec = ri.with_(MATRIX, state_dtype=state, input_dtype="bf16", philox_rounds=rounds, rand_seed=4321,
                    W=window, k_lo=1, k_hi=window, R=window + 3, hpg=2 if window > 8 else MATRIX.hpg)
    prob = ri.make_problem(spec, 2700 + window)
    m, H, dim, ds = prob.meta, spec.H, spec.dim, spec.dstate
    zero_hr, inf_hr, nan_hrc = (0, 3), (1, 5), (2, 9, 7)
    for l in range(spec.L):
        prob.A[l][inf_hr[0]] = 0.0   # no decay: code x 1e38 overflows whatever the prefix
        for b in range(spec.B):
            s_ = int(m.src[l, b])
            if s_ == spec.pad_slot_id:
                continue
            st = prob.state[l][s_]
            h, r = zero_hr
            st[(h * dim + r) * ds:(h * dim + r + 1) * ds] = 0
            for e in range(spec.R):
                prob.x[l][s_, (e * H + h) * dim + r] = 0
            h, r = inf_hr
            prob.scale[l][s_, h * dim + r] = 1e38
            st[(h * dim + r) * ds:(h * dim + r) * ds + 8] = 0x7E if state == "f8e4m3" else 100
            if state == "f8e4m3":
                h, r, c = nan_hrc
                st[(h * dim + r) * ds + c] = 0x7F
    say("special rows", state, rounds, "window", window)
    expected = oracle_result(prob)
    st_g, sc_g = check(prob, dev, expected)
    st_o, sc_o = expected[0], expected[1]
    # the special rows of every written destination, exactly
    for l in range(spec.L):
        for i in range(spec.B):
            b = int(m.active[i])
            if b < 0:
                break
            s_, d_ = int(m.src[l, b]), int(m.dst[l, b])
            if s_ == spec.pad_slot_id or d_ == spec.pad_slot_id or int(m.prefix[b]) == 0:
                continue
            for (h, r) in (zero_hr, inf_hr):
                row = slice((h * dim + r) * ds, (h * dim + r + 1) * ds)
                assert not st_g[l][d_, row].any(), f"layer {l} slot {d_} head {h} row {r}: codes not zero"
                assert sc_g[l][d_, h * dim + r] == 0.0, f"layer {l} slot {d_} head {h} row {r}: scale not 0"
            if state == "f8e4m3":
                # the NaN row: the other codes as the oracle's (its scale is
                # compared within 1e-5 above), the NaN element a NaN code
                # (its sign is not fixed, IEEE 754)
                h, r, c = nan_hrc
                at = (h * dim + r) * ds + c
                row = np.r_[(h * dim + r) * ds:at, at + 1:(h * dim + r + 1) * ds]
                assert np.array_equal(st_g[l][d_, row], st_o[l][d_, row]), f"layer {l} slot {d_}: NaN row differs"
                assert st_o[l][d_, at] == 0x7F and st_g[l][d_, at] & 0x7F == 0x7F


@pytest.mark.parametrize("state", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("window", [8, 16])
def test_wide_state_special_values(dev, state, window):
    """NaN and infinities in a source state of a wide dtype, through the whole
    kernel: the NaN element stays NaN (of either sign: IEEE 754 does not fix
    the sign of a NaN that arithmetic yields), each infinity stays the same
    infinity (the decay is positive and the added terms finite), and every
    other element is compared with the oracle as usual."""
    spec = ri.with_(MATRIX, state_dtype=state, input_dtype="bf16", W=window, k_lo=1, k_hi=window, R=window + 3,
                    hpg=2 if window > 8 else MATRIX.hpg)
    prob = ri.make_problem(spec, 2800 + window)
    m, dim, ds = prob.meta, spec.dim, spec.dstate
    nan, pinf, ninf = {"f32": (np.float32(np.nan), np.float32(np.inf), np.float32(-np.inf)),
                       "bf16": (0x7FC0, 0x7F80, 0xFF80),
                       "f16": (np.float16(np.nan), np.float16(np.inf), np.float16(-np.inf))}[state]
    spots = [((2, 9, 7), nan), ((1, 5, 3), pinf), ((1, 5, 4), ninf), ((7, 63, 127), pinf)]
    for l in range(spec.L):
        for b in range(spec.B):
            s_ = int(m.src[l, b])
            if s_ == spec.pad_slot_id:
                continue
            for (h, r, c), v in spots:
                prob.state[l][s_, (h * dim + r) * ds + c] = v
    say("wide special values", state, "window", window)
    expected = oracle_result(prob)
    st_g, _ = check(prob, dev, expected)
    st_o = expected[0]
    n_checked = 0
    for l in range(spec.L):
        for i in range(spec.B):
            b = int(m.active[i])
            if b < 0:
                break
            s_, d_ = int(m.src[l, b]), int(m.dst[l, b])
            if s_ == spec.pad_slot_id or d_ == spec.pad_slot_id or int(m.prefix[b]) == 0:
                continue
            for (h, r, c), v in spots[1:]:
                at = (h * dim + r) * ds + c
                assert st_o[l][d_, at].tobytes() == np.asarray(v, st_o[l].dtype).tobytes()
                assert st_g[l][d_, at].tobytes() == st_o[l][d_, at].tobytes(), \
                    f"layer {l} slot {d_} head {h} row {r} col {c}: infinity not kept"
            n_checked += 1
    assert n_checked > 0


def oracle_result(prob):
    import oracle
    return oracle.materialize(prob, want_exact=True)


@pytest.mark.parametrize("state", ["bf16", "f16", "i8", "f8e4m3"])
@pytest.mark.parametrize("rounds", [0, 10])
@pytest.mark.parametrize("dstate", [16, 128])
def test_debug_encode_rows_bit_exact(dev, state, rounds, dstate):
    """The kernel's encode step on arbitrary fp32 rows equals the oracle's,
    code for code (nearest-even and Philox stochastic rounding)."""
    import torch
    import oracle
    from replayssm_persistent_rssm_amd import rssm_debug_encode_rows
    if ri.one_byte(state) and dstate != 128:
        pytest.skip("one-byte state rows have 128 columns")
    rng = np.random.default_rng(3000 + dstate + rounds)
    n = 96
    rows = (rng.standard_normal((n, dstate)) * np.exp(rng.uniform(-12, 12, (n, 1)))).astype(np.float32)
    rows[0] = 0.0
    rows[1, :] = np.float32(1.0 + 2.0 ** -8)           # bf16 tie
    rows[2, :] = np.float32(2.0 ** -130)               # fp32 subnormal
    rows[3, :dstate // 2] = np.float32(70000.0)        # fp16 overflow / saturation
    rows[4] = rng.standard_normal(dstate).astype(np.float32) * 1e-8
    # row maxima at the edges of the short quotient sequences' range [2^-100, 2^100]
    for i, top in zip(range(5, 10), (2.0 ** 100, 2.0 ** -100, 2.0 ** -101, 2.0 ** 101, 3.0e38)):
        rows[i] = (rng.uniform(-1, 1, dstate) * top).astype(np.float32)
        rows[i, 7] = np.float32(top)
    coords = np.stack([rng.integers(0, 48, n), rng.integers(0, 256, n), rng.integers(0, 256, n),
                       rng.integers(0, 64, n)], 1).astype(np.int32)
    seed = 0x123456789ABCDEF
    spec = ri.with_(MATRIX, dstate=dstate, state_dtype=state, philox_rounds=rounds, rand_seed=seed)
    say("encode rows", state, rounds, dstate)
    t_rows = torch.from_numpy(rows).to(dev)
    t_coords = torch.from_numpy(coords).to(dev)
    t_seed = torch.tensor([seed], dtype=torch.int64, device=dev)
    eb = ri.ELEM_BYTES[state]
    out = torch.zeros((n, dstate * eb), dtype=torch.uint8, device=dev)
    scales = torch.zeros((n,), dtype=torch.float32, device=dev) if ri.one_byte(state) else None
    rssm_debug_encode_rows(t_rows, t_coords, t_seed if rounds else None, out, scales, state_dtype=state,
                           dstate=dstate, philox_rounds=rounds)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i in range(n):
        l, b, h, r = (int(v) for v in coords[i])
        codes, scale = oracle.encode_row(spec, rows[i], l, b, h, r)
        assert np.array_equal(got[i], codes.view(np.uint8)), f"row {i} ({l},{b},{h},{r})"
        if scales is not None:
            assert np.float32(scales[i].item()).view(np.uint32) == np.float32(scale).view(np.uint32), f"row {i} scale"


def test_row_scales_correctly_rounded(dev):
    """The one-byte encode's row scale m/qmax and inverse qmax/m equal IEEE
    fp32 division (numpy float32) bit for bit: every mantissa at exponents on
    both sides of the short sequences' range [2^-100, 2^100] and at the ends
    of the normal range, the first 2^20 subnormals, and special values.
    Inside the range the sequences only scale by powers of two with m (no
    operand nears the subnormal or overflow range), so every mantissa at one
    exponent stands for the whole range."""
    import torch
    from replayssm_persistent_rssm_amd import rssm_debug_row_scales
    mant = np.arange(1 << 23, dtype=np.uint32)
    parts = [((np.uint32(e + 127) << np.uint32(23)) | mant).view(np.float32)
             for e in (-126, -120, -101, -100, -1, 0, 99, 100, 127)]
    parts.append(np.arange(1, 1 << 20, dtype=np.uint32).view(np.float32))
    parts.append(np.array([0.0, 2.0 ** -100, 2.0 ** 100, np.finfo(np.float32).max, np.inf], np.float32))
    m = np.concatenate(parts)
    d_m = torch.from_numpy(m).to(dev)
    for state, q in (("i8", 127), ("f8e4m3", 448)):
        say("row scales", state, "values", m.size)
        scale = torch.empty_like(d_m)
        inv = torch.empty_like(d_m)
        rssm_debug_row_scales(d_m, scale, inv, state_dtype=state)
        torch.cuda.synchronize()
        with np.errstate(divide="ignore", over="ignore"):
            want_inv = np.float32(q) / m
            want_scale = m / np.float32(q)
        ok = (m > 0) & np.isfinite(m) & np.isfinite(want_inv)
        want_scale = np.where(ok, want_scale, np.float32(0)).astype(np.float32)
        got_s = scale.cpu().numpy()
        got_i = inv.cpu().numpy()
        bad_s = np.flatnonzero(got_s.view(np.uint32) != want_scale.view(np.uint32))
        assert bad_s.size == 0, f"{state}: {bad_s.size} scales differ, first m={m[bad_s[0]]!r}"
        bad_i = np.flatnonzero(ok & (got_i.view(np.uint32) != want_inv.view(np.uint32)))
        assert bad_i.size == 0, f"{state}: {bad_i.size} inverses differ, first m={m[bad_i[0]]!r}"


# --------------------------------------------------------------------------
# Full-size workloads, sampled (launch configuration of the benchmark)
# --------------------------------------------------------------------------
def _pool_snapshot(dp, slot_sets):
    """Byte copies (on the device) of the given slots of every layer's state
    and scale pools; slot_sets[l] is a sorted list of slots of layer l."""
    import torch
    snap = []
    for l, sl in enumerate(slot_sets):
        idx = torch.tensor(sl, dtype=torch.long, device=dp.state[l].device)
        st = dp.state[l].view(torch.uint8)[idx].clone() if sl else None
        sc = dp.scale[l].view(torch.uint8)[idx].clone() if (sl and dp.scale) else None
        snap.append((idx, st, sc))
    return snap


def _assert_snapshot_equal(dp, snap, what):
    import torch
    for l, (idx, st, sc) in enumerate(snap):
        if st is None:
            continue
        assert torch.equal(dp.state[l].view(torch.uint8)[idx], st), f"{what}: layer {l} state bytes changed"
        if sc is not None:
            assert torch.equal(dp.scale[l].view(torch.uint8)[idx], sc), f"{what}: layer {l} scale bytes changed"


def _assert_fill(dp, slot_sets, fill, what):
    """Every byte of the given slots (state and scale pools) is the fill byte."""
    import torch
    for l, sl in enumerate(slot_sets):
        if not sl:
            continue
        idx = torch.tensor(sl, dtype=torch.long, device=dp.state[l].device)
        assert bool((dp.state[l].view(torch.uint8)[idx] == fill).all().item()), f"{what}: layer {l} state written"
        if dp.scale:
            assert bool((dp.scale[l].view(torch.uint8)[idx] == fill).all().item()), f"{what}: layer {l} scale written"


def _sampled_full_size(dev, name, n_active, seed, n_samples=24, all_pad_after=False):
    """One call on the full-size problem in the benchmark's launch
    configuration.  Byte for byte: every slot of every layer outside the
    listed requests' destinations keeps its bytes (the drawn source range is
    compared with a device copy taken before the call; every other slot must
    still hold the fill byte).  Sampled: listed (request, layer, head) tiles
    against the oracle, tile by tile."""
    import torch
    import oracle
    import parity
    import rssm_harness as hx
    spec = ri.CONFIGS[name]
    say("full size", name, "n_active", n_active, "seed", seed)
    dp = ri.make_device_problem(spec, seed, dev, n_active=n_active)
    tabs = hx.tables(dp, dev)
    torch.cuda.synchronize()
    m = dp.meta
    listed = [int(v) for v in m.active[:n_active]]
    if n_active < spec.B:
        assert int(m.active[n_active]) == -1
    pad = spec.pad_slot_id
    # slots the generator drew (the source range), per layer; the rest holds 0xA5
    drawn = sorted(set(int(v) for v in m.src.reshape(-1) if v != pad))
    drawn = list(range(drawn[0], drawn[-1] + 1)) if drawn else []
    dst_of = [sorted(int(m.dst[l, b]) for b in listed if m.src[l, b] != pad and m.dst[l, b] != pad)
              for l in range(spec.L)]
    fill_slots = [sorted(set(range(m.slots)) - set(drawn) - set(dst_of[l])) for l in range(spec.L)]
    src_snap = _pool_snapshot(dp, [drawn] * spec.L)
    torch.cuda.synchronize()
    hx.materialize(dp, tabs)
    torch.cuda.synchronize()
    _assert_snapshot_equal(dp, src_snap, "source slots")
    _assert_fill(dp, fill_slots, 0xA5, "slot outside the listed destinations")

    if n_active:
        rng = np.random.default_rng(seed)
        n_tile = spec.dim * spec.dstate
        _, _, d_x, d_B, d_dt = ri.dense_sizes(spec)
        picks = [(0, 0, 0), (n_active - 1, spec.L - 1, spec.H - 1)]
        picks += [(int(rng.integers(n_active)), int(rng.integers(spec.L)), int(rng.integers(spec.H)))
                  for _ in range(n_samples)]
        np_dt = ri.STORAGE_NP[spec.state_dtype]
        for i, l, h in picks:
            b = int(m.active[i])
            s, d = int(m.src[l, b]), int(m.dst[l, b])
            k, r0 = int(m.prefix[b]), int(m.ring_start[b])

            def host(t, sl):
                a = t[sl].cpu()
                if a.dtype == torch.bfloat16:
                    a = a.view(torch.int16)
                return a.numpy()
            src_tile = host(dp.state[l], (s, slice(h * n_tile, (h + 1) * n_tile))).view(np_dt)
            gpu_tile = host(dp.state[l], (d, slice(h * n_tile, (h + 1) * n_tile))).view(np_dt)
            src_sc = gpu_sc = None
            if dp.scale:
                src_sc = host(dp.scale[l], (s, slice(h * spec.dim, (h + 1) * spec.dim)))
                gpu_sc = host(dp.scale[l], (d, slice(h * spec.dim, (h + 1) * spec.dim)))
            x_slot = host(dp.x[l], (s, slice(0, d_x))).view(ri.STORAGE_NP[spec.input_dtype])
            B_slot = host(dp.Bm[l], (s, slice(0, d_B))).view(ri.STORAGE_NP[spec.input_dtype])
            dt_slot = host(dp.dt[l], (s, slice(0, d_dt)))
            A_h = float(dp.A[l][h].item())
            codes, scale, exact, mag = oracle.tile(spec, l, b, h, r0, k, A_h, src_tile, src_sc, x_slot, B_slot,
                                                   dt_slot)
            what = f"{name} i={i} b={b} l={l} h={h} k={k}"
            if k == 0:
                assert np.array_equal(gpu_tile.view(np.uint8), src_tile.view(np.uint8)), what
                if gpu_sc is not None:
                    assert np.array_equal(gpu_sc.view(np.uint32), src_sc.view(np.uint32)), what
            else:
                parity.compare_tile(spec.state_dtype, gpu_tile, codes, exact, mag, gpu_sc, scale, what)
    if all_pad_after:
        # the same listed requests with every source slot the pad slot: the
        # launch (the benchmark's all-pad call) must leave every pool byte as
        # is -- the source range against its copy, the written destinations
        # against a copy taken now, everything else still the fill byte
        say("full size", name, "all listed, every source the pad slot")
        dst_snap = _pool_snapshot(dp, dst_of)
        pad_src = torch.full((spec.L, spec.B), pad, dtype=torch.int32, device=dev)
        hx.prepared(dp, hx.Tables(**{**tabs.__dict__, "src_slots": pad_src}))()
        torch.cuda.synchronize()
        _assert_snapshot_equal(dp, src_snap, "all-pad call: source slots")
        _assert_snapshot_equal(dp, dst_snap, "all-pad call: destination slots")
        _assert_fill(dp, fill_slots, 0xA5, "all-pad call: other slots")
        del dst_snap
    del src_snap, dp, tabs
    torch.cuda.empty_cache()
    return set(listed)


@pytest.mark.parametrize("n_active", [256, 16, 1, 0])
def test_full_size_large_bf16_sampled(dev, n_active):
    """The large bf16 workload at every active count of its sweep (256, 16,
    1, 0); a single request gets more sampled tiles."""
    _sampled_full_size(dev, "large_bf16", n_active, 1000 + 2 * 10 + n_active % 7,
                       n_samples=64 if n_active == 1 else 24, all_pad_after=n_active == 256)


def test_full_size_large_i8_sampled(dev):
    _sampled_full_size(dev, "large_i8", 64, 1003)


def test_full_size_large_f8sr_sampled(dev):
    _sampled_full_size(dev, "large_f8sr", 128, 1004)

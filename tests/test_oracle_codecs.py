"""Oracle number formats and rounding, pinned to library casts and exhaustive
code tables.

Round to nearest even is checked against torch's CPU casts (bf16, fp16, OCP
e4m3fn) on in-range values; decode against torch's casts of every code; the
int8 grid against numpy's rint.  Stochastic rounding (the library's own
reading: round the magnitude up iff u < f * 2^32) is checked at its exact
thresholds and for unbiasedness.
"""
import numpy as np
import pytest
import torch

FMT = {"bf16": (torch.bfloat16, torch.int16, 0xFFFF), "f16": (torch.float16, torch.int16, 0xFFFF),
       "f8e4m3": (torch.float8_e4m3fn, torch.uint8, 0xFF)}


def torch_codes(dtype, vals):
    tdt, view, mask = FMT[dtype]
    t = torch.from_numpy(np.asarray(vals, np.float32)).to(tdt).view(view)
    return (t.numpy().astype(np.int64) & mask).astype(np.uint32)


def all_codes(dtype):
    n = 1 << 16 if dtype in ("bf16", "f16") else 256
    return np.arange(n, dtype=np.uint32)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f8e4m3"])
def test_decode_every_code_matches_torch(orc, dtype):
    codes = all_codes(dtype)
    tdt, view, _ = FMT[dtype]
    raw = codes.astype(np.uint16 if view == torch.int16 else np.uint8)
    ref = torch.from_numpy(raw.view(np.int16) if view == torch.int16 else raw).view(tdt).to(torch.float64).numpy()
    got = orc.decode(dtype, raw)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), codes[~same][:10]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f8e4m3"])
def test_every_finite_code_round_trips(orc, dtype):
    codes = all_codes(dtype)
    raw = codes.astype(np.uint16 if dtype != "f8e4m3" else np.uint8)
    vals = orc.decode(dtype, raw)
    for c, v in zip(codes, vals):
        if np.isnan(v) or np.isinf(v):
            continue
        assert orc.round_value(dtype, np.float32(v)) == c
        assert orc.round_value(dtype, np.float32(v), True, 0) == c
        assert orc.round_value(dtype, np.float32(v), True, 0xFFFFFFFF) == c


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f8e4m3"])
def test_nearest_even_matches_torch(orc, dtype):
    rng = np.random.default_rng(11)
    maxv = {"bf16": 3.3e38, "f16": 65504.0, "f8e4m3": 448.0}[dtype]
    tiny = {"bf16": 1e-38, "f16": 6e-8, "f8e4m3": 2.0**-9}[dtype]
    vals = np.concatenate([rng.standard_normal(3000), rng.standard_normal(1500) * tiny * 8,
                           rng.uniform(-maxv, maxv, 1500)]).astype(np.float32)
    # ties: midpoints of neighbouring positive codes, representable in fp32
    pos = np.arange(1, {"bf16": 0x7F7F, "f16": 0x7BFF, "f8e4m3": 0x7E}[dtype], 37, dtype=np.uint32)
    raw = pos.astype(np.uint16 if dtype != "f8e4m3" else np.uint8)
    lo = orc.decode(dtype, raw)
    hi = orc.decode(dtype, (pos + 1).astype(raw.dtype))
    mids = ((lo + hi) / 2).astype(np.float32)
    exact_mid = mids.astype(np.float64) == (lo + hi) / 2
    vals = np.concatenate([vals, mids[exact_mid], -mids[exact_mid]])
    ref = torch_codes(dtype, vals)
    got = np.array([orc.round_value(dtype, v) for v in vals], np.uint32)
    bad = got != ref
    assert not bad.any(), list(zip(vals[bad][:5], got[bad][:5], ref[bad][:5]))
    # NaN of either sign: torch's fp16 and e4m3 casts keep the sign, as the
    # oracle does; its bf16 cast returns 0xFFFF for both, so there only the
    # NaN-ness is compared (the sign of a converted NaN is unspecified)
    nans = np.array([np.float32("nan"), -np.float32("nan")], np.float32)
    got_nan = np.array([orc.round_value(dtype, v) for v in nans], np.uint32)
    assert np.isnan(orc.decode(dtype, got_nan.astype(raw.dtype))).all()
    if dtype != "bf16":
        np.testing.assert_array_equal(got_nan, torch_codes(dtype, nans))


def test_bf16_f16_overflow_to_infinity(orc):
    # IEEE nearest-even overflow, as torch's casts do.
    for dtype in ("bf16", "f16"):
        top = {"bf16": 3.3895314e38, "f16": 65504.0}[dtype]
        vals = np.array([top, np.nextafter(np.float32(top), np.float32(np.inf)), np.inf, -np.inf,
                         65519.0, 65520.0, 65535.0, -65520.0], np.float64).astype(np.float32)
        ref = torch_codes(dtype, vals)
        got = np.array([orc.round_value(dtype, v) for v in vals], np.uint32)
        np.testing.assert_array_equal(got, ref)


def test_e4m3_saturates(orc):
    assert orc.round_value("f8e4m3", 448.0) == 0x7E
    assert orc.round_value("f8e4m3", 500.0) == 0x7E
    assert orc.round_value("f8e4m3", -1e9) == 0xFE
    assert orc.round_value("f8e4m3", 500.0, True, 0) == 0x7E


def test_int8_grid_matches_rint(orc):
    rng = np.random.default_rng(3)
    t = np.concatenate([rng.uniform(-130, 130, 4000), np.arange(-130, 131) + 0.5,
                        np.arange(-130, 131) - 0.5, np.arange(-3, 4, 0.25)]).astype(np.float32)
    ref = np.clip(np.rint(t.astype(np.float64)), -127, 127).astype(np.int64)
    got = np.array([orc.round_value("i8", v) for v in t], np.int64)
    got = np.where(got >= 128, got - 256, got)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f8e4m3", "i8"])
def test_stochastic_threshold_is_exact(orc, dtype):
    # v between grid points lo < v < hi with f = (v - lo)/(hi - lo): up iff u < f * 2^32.
    cases = {"bf16": (1.0, 1.0 + 2**-7), "f16": (1.0, 1.0 + 2**-10), "f8e4m3": (1.0, 1.125), "i8": (3.0, 4.0)}
    lo, hi = cases[dtype]
    for f in (0.25, 0.5, 0.75, 1 / 3):
        v = np.float32(lo + f * (hi - lo))
        fe = (float(v) - lo) / (hi - lo)
        thr = fe * 2**32
        down = orc.round_value(dtype, lo)
        up = orc.round_value(dtype, hi)
        u_last_up = int(np.ceil(thr)) - 1
        assert orc.round_value(dtype, v, True, u_last_up) == up
        assert orc.round_value(dtype, v, True, u_last_up + 1) == down
        assert orc.round_value(dtype, v, True, 0) == up
        assert orc.round_value(dtype, v, True, 0xFFFFFFFF) == down
        # sign symmetry
        assert orc.round_value(dtype, -v, True, u_last_up) == orc.round_value(dtype, -hi)


def test_stochastic_saturates(orc):
    assert orc.round_value("bf16", np.float32(3.3961e38), True, 0) == 0x7F7F
    assert orc.round_value("f16", 65519.0, True, 0) == 0x7BFF
    assert orc.round_value("f16", 70000.0, True, 0) == 0x7BFF
    assert orc.round_value("i8", 130.0, True, 0) == 127


def test_stochastic_rounding_is_unbiased_over_seeds(orc):
    """Mean of SR(v) over 4096 seeds is v within 3 sigma, through the full
    row encode with Philox4x32-10 words."""
    import rssm_inputs as ri
    spec = ri.with_(ri.CONFIGS["tiny_f32"], dstate=16, state_dtype="bf16")
    rng = np.random.default_rng(5)
    row = rng.standard_normal(16).astype(np.float32)
    acc = np.zeros(16)
    n = 4096
    for s in range(n):
        codes, _ = orc.encode_row(spec, row, 0, 1, 2, 3, state_dtype="bf16", philox_rounds=10, seed=s * 7919 + 1)
        acc += orc.decode("bf16", codes)
    mean = acc / n
    # per element: SR variance = (v-lo)(hi-v) <= ulp^2 / 4
    ulp = 2.0 ** (np.floor(np.log2(np.abs(row.astype(np.float64)))) - 7)
    sigma = ulp / 2 / np.sqrt(n)
    assert np.all(np.abs(mean - row) <= 3 * sigma + 1e-12)


def test_zero_rounds_is_nearest_even(orc):
    import rssm_inputs as ri
    spec = ri.with_(ri.CONFIGS["tiny_f32"], dstate=16)
    rng = np.random.default_rng(6)
    row = rng.standard_normal(16).astype(np.float32)
    for dt in ("bf16", "f16"):
        codes, _ = orc.encode_row(spec, row, 0, 0, 0, 0, state_dtype=dt, philox_rounds=0, seed=99)
        np.testing.assert_array_equal(codes.view(np.uint16).astype(np.uint32), torch_codes(dt, row))


def test_row_quantization_e3_e4(orc):
    """One-byte rows: scale = rowmax/qmax, codes reconstruct the row within
    half a quantum (nearest) or one quantum (stochastic)."""
    import rssm_inputs as ri
    spec = ri.CONFIGS["tiny_f32"]
    rng = np.random.default_rng(8)
    for dt, qmax in (("i8", 127.0), ("f8e4m3", 448.0)):
        for rounds in (0, 10):
            row = (rng.standard_normal(16) * 3).astype(np.float32)
            codes, scale = orc.encode_row(spec, row, 0, 0, 0, 0, state_dtype=dt, philox_rounds=rounds, seed=17)
            assert scale == np.float32(np.abs(row).max()) / np.float32(qmax)
            deq = orc.decode(dt, codes) * scale
            t = row.astype(np.float64) / scale
            # grid spacing around t
            if dt == "i8":
                q = np.ones_like(t)
            else:
                q = 2.0 ** (np.maximum(np.floor(np.log2(np.maximum(np.abs(t), 2.0**-9))), -6) - 3)
            bound = (0.5 if rounds == 0 else 1.0) * q * scale * (1 + 1e-6) + 1e-30
            assert np.all(np.abs(deq - row) <= bound)
            # the largest magnitude maps to the top code
            top = np.argmax(np.abs(row))
            assert abs(orc.decode(dt, codes[top:top + 1])[0]) == qmax
    zero = np.zeros(16, np.float32)
    codes, scale = orc.encode_row(spec, zero, 0, 0, 0, 0, state_dtype="i8", philox_rounds=0)
    assert scale == 0.0 and not codes.any()


def test_nan_element_in_one_byte_row(orc):
    """A NaN element takes no part in a one-byte row's quantization: the row
    scale and every other code equal those of the same row with that element
    set to 0, with nearest-even and with stochastic rounding (each element's
    random word depends on its own coordinates only).  The NaN element itself
    takes the codes the design reads for it: 0 for int8, S.1111.111 (its own
    sign) for e4m3."""
    import rssm_inputs as ri
    spec = ri.CONFIGS["tiny_f32"]
    rng = np.random.default_rng(21)
    for dt in ("i8", "f8e4m3"):
        for rounds in (0, 10):
            for sign in (1.0, -1.0):
                row = (rng.standard_normal(16) * 3).astype(np.float32)
                ref_row = row.copy()
                ref_row[5] = 0.0
                row[5] = np.copysign(np.float32("nan"), np.float32(sign))   # (a product would keep +NaN)
                codes, scale = orc.encode_row(spec, row, 1, 2, 3, 4, state_dtype=dt, philox_rounds=rounds, seed=29)
                ref, ref_scale = orc.encode_row(spec, ref_row, 1, 2, 3, 4, state_dtype=dt, philox_rounds=rounds,
                                                seed=29)
                assert scale == ref_scale and scale > 0
                keep = np.arange(16) != 5
                np.testing.assert_array_equal(np.asarray(codes)[keep], np.asarray(ref)[keep])
                nan_code = int(np.asarray(codes).view(np.uint8)[5])
                assert nan_code == (0 if dt == "i8" else (0xFF if sign < 0 else 0x7F))

"""The comparison rules of the GPU parity tests (tests/parity.py), on planted
codes (no GPU): NaN placement is exact and its sign free, the one-step and
one-ulp tolerances hold and reject a two-step difference, an infinity
compares equal to itself."""
import numpy as np
import pytest

import parity


def _tile(dtype, codes, exact):
    codes = np.asarray(codes, {"f8e4m3": np.uint8, "bf16": np.uint16, "f16": np.uint16,
                               "f32": np.float32, "i8": np.int8}[dtype])
    exact = np.asarray(exact, np.float64)
    return codes, exact, np.maximum(np.abs(exact), 1.0)


def _cmp(dtype, got, exp_codes, exact):
    e, x, m = _tile(dtype, exp_codes, exact)
    g, _, _ = _tile(dtype, got, exact)
    parity.compare_tile(dtype, g, e, x, m, what="planted")


def test_e4m3_nan_sign_is_free_and_placement_exact():
    exact = [1.0, np.nan, 2.0]
    _cmp("f8e4m3", [0x38, 0xFF, 0x40], [0x38, 0x7F, 0x40], exact)
    _cmp("f8e4m3", [0x38, 0x7F, 0x40], [0x38, 0x7F, 0x40], exact)
    with pytest.raises(AssertionError, match="1 NaN in the oracle only, 0 on"):
        _cmp("f8e4m3", [0x38, 0x7E, 0x40], [0x38, 0x7F, 0x40], exact)        # 448, one step from the NaN code
    with pytest.raises(AssertionError, match="0 NaN in the oracle only, 1 on the GPU only"):
        _cmp("f8e4m3", [0x38, 0x7F, 0x40], [0x38, 0x7E, 0x40], [1.0, 448.0, 2.0])


def test_one_byte_step_tolerance():
    _cmp("f8e4m3", [0x39, 0x3F], [0x38, 0x40], [1.0, 2.0])
    _cmp("f8e4m3", [0x80, 0x01], [0x00, 0x00], [0.0, 0.0])                    # -0 and +0 are one position
    with pytest.raises(AssertionError, match="more than one step"):
        _cmp("f8e4m3", [0x3A], [0x38], [1.0])
    _cmp("i8", [5, -4], [4, -4], [4.0, -4.0])
    with pytest.raises(AssertionError, match="more than one step"):
        _cmp("i8", [6], [4], [4.0])


def test_bf16_nan_sign_and_payload_free_inf_kept():
    _cmp("bf16", [0x3F80, 0xFFC1, 0x7F80], [0x3F80, 0x7FC0, 0x7F80], [1.0, np.nan, np.inf])
    with pytest.raises(AssertionError, match="1 NaN in the oracle only, 0 on"):
        _cmp("bf16", [0x3F80, 0x7F80], [0x3F80, 0x7FC0], [1.0, np.nan])       # inf for a NaN
    with pytest.raises(AssertionError, match="off by more than 1 ulp"):
        _cmp("bf16", [0x3F82], [0x3F80], [1.0])


def test_f16_nan_free_sign():
    _cmp("f16", [0x3C00, 0xFE00], [0x3C00, 0x7E00], [1.0, np.nan])
    with pytest.raises(AssertionError, match="0 NaN in the oracle only, 1 on the GPU only"):
        _cmp("f16", [0x7E00], [0x7C00], [np.inf])


def test_f32_infinity_and_nan():
    _cmp("f32", [1.0, np.inf, -np.inf, np.nan], [1.0, np.inf, -np.inf, np.nan], [1.0, np.inf, -np.inf, np.nan])
    with pytest.raises(AssertionError, match="beyond 1e-5"):
        _cmp("f32", [1.0, -np.inf], [1.0, np.inf], [1.0, np.inf])
    with pytest.raises(AssertionError, match="0 NaN in the oracle only, 1 on the GPU only"):
        _cmp("f32", [np.nan], [1.0], [1.0])
    with pytest.raises(AssertionError, match="beyond 1e-5"):
        _cmp("f32", [1.0 + 3e-5], [1.0], [1.0])


def test_opposite_infinity_rejected_in_two_byte_state():
    with pytest.raises(AssertionError, match="off by more than 1 ulp"):
        _cmp("bf16", [0xFF80], [0x7F80], [np.inf])
    with pytest.raises(AssertionError, match="off by more than 1 ulp"):
        _cmp("f16", [0x7BFF], [0x7C00], [np.inf])        # largest finite for an input infinity

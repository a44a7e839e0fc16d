"""CPU checks of the element-wise comparison the GPU parity tests use
(tests/mxgpu.py): each rule is exercised on hand-made values, so a plausible
mistake in it (a sign test dropped, the overflow exemption applied
everywhere, the subnormal floor too wide) fails here."""
import numpy as np

from mxgpu import BF16_MAX, FP32_OVERFLOW, TOL_ABS, compare


def bits(x):
    """float64 values -> bf16 bit patterns (truncation is enough here: the
    values below are exact bf16 numbers)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_ordinary_tolerance():
    ref = np.array([1.0, 1.0, -3.0])
    mag = np.array([1.0, 1.0, 3.0])
    assert compare(bits([1.0, 1.0078125, -3.0]), ref, mag)[0] == 0
    assert compare(bits([1.0, 1.03125, -3.0]), ref, mag)[0] == 1  # 2^-5 off


def test_nan_must_match_nan():
    ref = np.array([np.nan, 2.0])
    mag = np.array([np.nan, 2.0])
    assert compare(bits([np.nan, 2.0]), ref, mag)[0] == 0
    assert compare(bits([1.0, 2.0]), ref, mag)[0] == 1          # NaN lost
    assert compare(bits([np.nan, np.nan]), ref, mag)[0] == 1    # NaN invented


def test_infinity_follows_the_oracles_rounding():
    # beyond the largest bf16 but inside the fp32 range: no partial sum can
    # overflow, the fp32 result rounds to the infinity of its own sign
    big = 3.4e38
    ref = np.array([big, -big])
    mag = np.array([big, big])
    assert compare(bits([np.inf, -np.inf]), ref, mag)[0] == 0
    assert compare(bits([-np.inf, -np.inf]), ref, mag)[0] == 1  # wrong sign
    assert compare(bits([BF16_MAX, -np.inf]), ref, mag)[0] == 1  # finite where the oracle overflows


def test_subnormal_floor_is_one_spacing():
    ref = np.array([2.0 ** -137, 3 * 2.0 ** -133])
    mag = ref.copy()
    assert compare(bits([0.0, 3 * 2.0 ** -133]), ref, mag)[0] == 0
    assert compare(bits([0.0, 2.0 ** -130]), ref, mag)[0] == 1  # 5 spacings off
    assert TOL_ABS == 2.0 ** -133


def test_fp32_overflow_exemption_needs_a_large_magnitude_sum():
    ref = np.array([1.0e38, 1.0e38])
    mag = np.array([FP32_OVERFLOW, 1.0e38])
    # a partial sum can overflow only in the first element
    assert compare(bits([np.inf, 1.0e38]), ref, mag)[0] == 0
    assert compare(bits([np.nan, 1.0e38]), ref, mag)[0] == 0
    assert compare(bits([1.0e38, np.inf]), ref, mag)[0] == 1
    assert compare(bits([1.0e38, np.nan]), ref, mag)[0] == 1
    # an overflowing partial sum fixes the sign of the infinity
    assert compare(bits([-np.inf]), np.array([2.0 ** 130]), np.array([2.0 ** 140]))[0] == 0
    assert compare(bits([-np.inf]), np.array([3.4e38]), np.array([3.4e38]))[0] == 1
    # alpha scales the accumulator before the bf16 rounding
    assert compare(bits([1.0e38, np.inf]), ref, np.array([1.0e38, 2.0e38]), alpha=2.0)[0] == 0

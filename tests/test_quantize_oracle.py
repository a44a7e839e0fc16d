"""Pins for the oracle's bf16 -> MXFP4 activation quantizer.

The pages define the E2M1 and E8M0 encodings but not how a scale is chosen;
the oracle follows the OCP MX v1.0 conversion rule (readings Q1-Q4 in
oracle/mxfp4_oracle.c).  Every check here states its expectation
independently of the oracle's code: hand-written values for the scale
choice and for each rounding tie, exact round trips of values that lie on
the scaled E2M1 grid, the half-spacing error bound of round-to-nearest,
sign symmetry, and the special blocks.
"""
import numpy as np
import pytest

import oracle

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # OCP E2M1 magnitudes, codes 0..7


def bf16_bits(x):
    """float -> bf16 bit pattern, exactly (x must be representable)."""
    f = np.array(x, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def bits_to_float(h):
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def codes(A, K):
    """Unpack [M, K/2] bytes into [M, K] codes (low nibble = even k)."""
    lo, hi = A & 0xF, A >> 4
    out = np.empty((A.shape[0], K), dtype=np.uint8)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return out


def dequant(A, S, K):
    c = codes(A, K)
    mag = np.array(E2M1)[c & 7]
    val = np.where(c & 8, -mag, mag)
    scale = np.where(S == 255, np.nan, np.ldexp(1.0, S.astype(np.int64) - 127))
    return val * np.repeat(scale, 32, axis=1)


def quant_block(values):
    X = bf16_bits(np.array(values, dtype=np.float64)).reshape(1, 32)
    A, S = oracle.quantize_mxfp4(X)
    return codes(A, 32)[0], int(S[0, 0])


@pytest.mark.parametrize("amax, scale_code", [
    (6.0, 127), (4.0, 127), (7.5, 127),        # max in [4, 8): X = 0
    (1.0, 125), (1.5, 125), (2.0, 126),        # floor(log2) - 2 + 127
    (448.0, 133), (0.09375, 121), (2.0 ** 100, 225),
    (2.0 ** -125, 0), (2.0 ** -130, 0),        # clamped at X = -127
    (1.5 * 2.0 ** 127, 252),                   # largest bf16 binade: 2^127 -> X = 125
])
def test_scale_exponent_rule(amax, scale_code):
    vals = [0.0] * 32
    vals[5] = amax
    vals[17] = -amax / 2
    _, s = quant_block(vals)
    assert s == scale_code


# Values scaled to X = 0 (the block max 6 fixes the scale), with the code
# round-to-nearest-even on the E2M1 grid gives: ties go to the even mantissa.
TIES = [
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
    (0.2421875, 0), (0.2578125, 1), (0.7421875, 1), (2.515625, 5), (4.96875, 6), (5.03125, 7),
    (6.0, 7), (6.5, 7), (7.0, 7), (7.96875, 7),  # saturation
]


@pytest.mark.parametrize("v, code", TIES)
def test_rounding_ties_and_saturation(v, code):
    vals = [6.0] + [0.0] * 31
    vals[9] = v
    vals[10] = -v
    c, s = quant_block(vals)
    assert s == 127
    assert c[9] == code
    assert c[10] == code | 8


def test_grid_values_round_trip_exactly():
    rng = np.random.default_rng(11)
    for _ in range(200):
        x = int(rng.integers(-120, 120))
        mags = rng.choice(E2M1, size=32)
        mags[rng.integers(0, 32)] = rng.choice([4.0, 6.0])  # pins the block max to [4, 8)
        signs = np.where(rng.random(32) < 0.5, -1.0, 1.0)
        vals = signs * mags * 2.0 ** x
        X = bf16_bits(vals).reshape(1, 32)
        A, S = oracle.quantize_mxfp4(X)
        assert int(S[0, 0]) == x + 127
        back = dequant(A, S, 32)[0]
        assert np.array_equal(back, vals), "grid values must survive quantization exactly"


def test_error_bound_on_random_blocks():
    """Round to nearest: |q - v| is at most half the local grid spacing
    (0.5 below 2, 1 in [2, 4), 2 in [4, 6]) times the scale; values the
    scale cannot reach (|v| > 6 * scale) saturate to 6 * scale."""
    rng = np.random.default_rng(12)
    M, K = 64, 256
    X = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-20, 20, (M, 1)))).astype(np.float32)
    Xb = (X.view(np.uint32) >> 16).astype(np.uint16)  # truncate to bf16
    x = bits_to_float(Xb)
    A, S = oracle.quantize_mxfp4(Xb)
    q = dequant(A, S, K)
    scale = np.repeat(np.ldexp(1.0, S.astype(np.int64) - 127), 32, axis=1)
    v = np.abs(x) / scale
    half = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    sat = v > 6.0
    err = np.abs(q - x) / scale
    assert np.all(err[~sat] <= half[~sat])
    assert np.all(np.abs(q[sat]) == 6.0 * scale[sat])
    # the scale of every block is 2^(floor(log2 amax) - 2)
    amax = np.abs(x).reshape(M, K // 32, 32).max(axis=2)
    assert np.array_equal(S.astype(np.int64) - 127, np.floor(np.log2(amax)).astype(np.int64) - 2)


def test_sign_symmetry():
    rng = np.random.default_rng(13)
    X = (rng.standard_normal((8, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    A1, S1 = oracle.quantize_mxfp4(X)
    A2, S2 = oracle.quantize_mxfp4(X ^ np.uint16(0x8000))
    assert np.array_equal(S1, S2)
    assert np.array_equal(codes(A1, 128) ^ 8, codes(A2, 128))


def test_special_blocks():
    nan, inf = float("nan"), float("inf")
    c, s = quant_block([1.0] * 31 + [nan])
    assert s == 0xFF and not c.any()
    c, s = quant_block([-inf] + [1.0] * 31)
    assert s == 0xFF and not c.any()
    c, s = quant_block([0.0] * 32)
    assert s == 0 and not c.any()
    c, s = quant_block([-0.0] + [0.0] * 31)
    assert s == 0 and c[0] == 8 and not c[1:].any()
    # a negative value far below the block max rounds to -0
    c, s = quant_block([6.0, -0.125] + [0.0] * 30)
    assert s == 127 and c[1] == 8


def test_layout_strides_and_rows():
    """Row r, block kb of X lands in bytes [r, kb*16 : kb*16+16] and scale
    [r, kb]; a padded input pitch changes nothing."""
    rng = np.random.default_rng(14)
    M, K = 5, 96
    X = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    A, S = oracle.quantize_mxfp4(X)
    Xp = np.full((M, K + 40), 0x7FC0, dtype=np.uint16)  # NaN padding must not be read
    Xp[:, :K] = X
    Ap, Sp = oracle.quantize_mxfp4(Xp, K, ldx=K + 40)
    assert np.array_equal(A, Ap) and np.array_equal(S, Sp)
    for r in range(M):
        for kb in range(K // 32):
            a1, s1 = oracle.quantize_mxfp4(X[r:r + 1, kb * 32:(kb + 1) * 32])
            assert np.array_equal(a1[0], A[r, kb * 16:(kb + 1) * 16]) and s1[0, 0] == S[r, kb]

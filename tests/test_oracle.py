"""Pins for the CPU oracle, each against something other than the oracle.

- code tables: the pages' printed values (tests/golden/mx_codes.txt) and the
  OCP bit-field definitions of E2M1 and E8M0;
- bf16 rounding: torch's float32 -> bfloat16 conversion (a library routine)
  and closed-form cases where rounding twice would differ;
- the GEMM: the identity-matrix test of the GEMM tutorial page ("Optimizing
  GEMM in HIP": B = I implies the product equals A), exact rational brute
  force (Python Fractions), numpy's float64 matmul on inputs whose sums are
  exact in float64, and algebraic invariants (linearity, sign, scale,
  transpose, block permutation).
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from block_scaled_precision_mxfp4_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent definitions used only as pins


def e2m1_bitfield(code: int) -> float:
    """OCP E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no
    inf/NaN; exponent field 0 is subnormal: 2^0 * (m/2)."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m / 2.0) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
    return -mag if s else mag


def e8m0_as_fp32_exponent(e: int) -> float:
    """E8M0 1..254 is the fp32 number with exponent field e and zero mantissa."""
    return struct.unpack("<f", struct.pack("<I", (e & 0xFF) << 23))[0]


def unpack_codes_np(X: np.ndarray, K: int) -> np.ndarray:
    """[rows, K/2] bytes -> [rows, K] codes; element 2i is the low nibble."""
    out = np.empty((X.shape[0], K), dtype=np.uint8)
    out[:, 0::2] = X[:, : K // 2] & 0x0F
    out[:, 1::2] = X[:, : K // 2] >> 4
    return out


def dequant_np(X: np.ndarray, SX: np.ndarray, K: int) -> np.ndarray:
    codes = unpack_codes_np(X, K)
    table = np.array([e2m1_bitfield(c) for c in range(16)], dtype=np.float64)
    vals = table[codes]
    sc = np.array([e8m0_as_fp32_exponent(e) if 0 < e < 255 else
                   (2.0 ** -127 if e == 0 else np.nan) for e in range(256)], dtype=np.float64)
    return vals * np.repeat(sc[SX[:, : K // 32]], 32, axis=1)


def frac_value(code: int, e: int) -> Fraction:
    s, ex, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if ex == 0 else Fraction(2) ** (ex - 1) * (1 + Fraction(m, 2))
    v = mag * Fraction(2) ** (e - 127)
    return -v if s else v


def rne_bf16_fraction(x: Fraction) -> int:
    """bf16 bits of the exact rational x, round to nearest, ties to even."""
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a == 0:
        return sign
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    while Fraction(2) ** (E + 1) <= a:
        E += 1
    Eq = max(E, -126)
    q = Fraction(2) ** (Eq - 7)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * q
    if v > Fraction(2) ** 127 * (2 - Fraction(1, 128)):
        return sign | 0x7F80
    bits = struct.unpack("<I", struct.pack("<f", float(v)))[0]
    return sign | (bits >> 16)


def small_problem(M, N, K, seed, e=(123, 131), dist="uniform", beta=0.0, c_sigma=None):
    return inputs.make_problem(M, N, K, seed=seed, dist=dist, e=e, beta=beta, c_sigma=c_sigma)


# ---------------------------------------------------------------------------
# code tables


def _golden_codes():
    rows = []
    with open(os.path.join(GOLDEN, "mx_codes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, code, val = line.split()
            rows.append((kind, int(code, 16), float(val)))
    return rows


def test_codes_match_page_table():
    rows = _golden_codes()
    assert sum(1 for r in rows if r[0] == "e2m1") == 16
    for kind, code, val in rows:
        got = oracle.e2m1(code) if kind == "e2m1" else oracle.e8m0(code)
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (kind, code)


def test_e2m1_matches_ocp_bitfields():
    for code in range(16):
        a, b = oracle.e2m1(code), e2m1_bitfield(code)
        assert a == b and math.copysign(1, a) == math.copysign(1, b), code


def test_e8m0_matches_fp32_exponent_field():
    for e in range(1, 255):
        assert oracle.e8m0(e) == e8m0_as_fp32_exponent(e), e
    assert math.isnan(oracle.e8m0(255))
    # code 0: reading adopted where the page contradicts itself (formula 2^(e-127))
    assert oracle.e8m0(0) == 2.0 ** -127


def test_nibble_order_low_is_even():
    X = np.array([[0x2A]], dtype=np.uint8)  # low nibble 0xA, high nibble 0x2
    assert oracle.fp4_code(X, 2, 0, 0) == 0xA
    assert oracle.fp4_code(X, 2, 0, 1) == 0x2


# ---------------------------------------------------------------------------
# bf16 rounding


def test_bf16_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    # add structured cases: exact ties, values next to ties, subnormals, max
    extra = []
    for base in (0x3F800000, 0x3F810000, 0x00010000, 0x00800000, 0x7F7F0000, 0x80018000):
        for d in (-1, 0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
            extra.append((base + d) & 0xFFFFFFFF)
    bits = np.concatenate([bits, np.array(extra, dtype=np.uint32)])
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_rne(float(x)) for x in f], dtype=np.uint16)
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(hex(bits[i]), hex(ref[i]), hex(got[i])) for i in bad[:5]]


def test_bf16_rounds_once_from_double():
    # 1 + 2^-8 + 2^-30: above the midpoint between 1 and 1 + 2^-7, so one
    # rounding gives 1 + 2^-7 (0x3F81); rounding through fp32 first would
    # land exactly on the midpoint and then tie to even (0x3F80).
    assert oracle.bf16_rne(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert oracle.bf16_rne(1.0 + 2.0 ** -8) == 0x3F80           # exact tie -> even
    assert oracle.bf16_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82       # tie -> even (up)
    assert oracle.bf16_rne(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == 0xBF81
    # overflow: the midpoint between the largest finite bf16 and 2^128 ties to
    # even, i.e. up to infinity; just below it stays finite
    mx = (2 - 2.0 ** -7) * 2.0 ** 127
    mid = (2 - 2.0 ** -8) * 2.0 ** 127
    assert oracle.bf16_rne(mx) == 0x7F7F
    assert oracle.bf16_rne(mid) == 0x7F80
    assert oracle.bf16_rne(mid * (1 - 2.0 ** -40)) == 0x7F7F
    # subnormals: spacing 2^-133
    assert oracle.bf16_rne(2.0 ** -133) == 0x0001
    assert oracle.bf16_rne(2.0 ** -134) == 0x0000                # tie -> even (0)
    assert oracle.bf16_rne(3 * 2.0 ** -134) == 0x0002            # tie -> even (2)
    assert oracle.bf16_rne(float("nan")) & 0x7FFF == 0x7FC0
    assert oracle.bf16_rne(-0.0) == 0x8000
    for x in (1.5, -3.0, 2.0 ** -126, 2.0 ** 127, 0.1):
        assert oracle.bf16_rne(x) == rne_bf16_fraction(Fraction(x))


# ---------------------------------------------------------------------------
# the GEMM


def _gemm(p, rows=None, cols=None):
    return oracle.mxgemm(p["A"], p["SA"], p["B"], p["SB"], p["K"], p["alpha"], p["beta"],
                         p["C"], rows=rows, cols=cols)


def test_identity_gives_dequantized_A():
    """B = I (code 0x2 = 1.0 on the diagonal), unit scales: D = bf16(A)."""
    M, K = 128, 512
    p = small_problem(M, K, K, seed=11)
    B = np.zeros((K, K // 2), dtype=np.uint8)
    for j in range(K):
        B[j, j // 2] |= (0x2 << 4) if (j & 1) else 0x2
    p["B"], p["SB"] = B, np.full((K, K // 32), 127, dtype=np.uint8)
    ref, mag, dref = _gemm(p)
    A = dequant_np(p["A"], p["SA"], K)
    assert np.array_equal(ref, A)
    expect = np.array([[rne_bf16_fraction(Fraction(float(v))) for v in row] for row in A],
                      dtype=np.uint16)
    # -0 * 1 + (+0) ... = +0 in the sum; compare values with +-0 equal
    same = (dref == expect) | (((dref | expect) & 0x7FFF) == 0)
    assert same.all()
    assert np.array_equal(mag, np.abs(A))


@pytest.mark.parametrize("K,e", [(32, (120, 134)), (64, (123, 131)), (96, (110, 140))])
def test_brute_force_fractions(K, e):
    M, N = 3, 4
    p = small_problem(M, N, K, seed=100 + K, e=e)
    ca, cb = unpack_codes_np(p["A"], K), unpack_codes_np(p["B"], K)
    ref, mag, dref = _gemm(p)
    for i in range(M):
        for j in range(N):
            exact = sum(frac_value(int(ca[i, k]), int(p["SA"][i, k // 32])) *
                        frac_value(int(cb[j, k]), int(p["SB"][j, k // 32])) for k in range(K))
            emag = sum(abs(frac_value(int(ca[i, k]), int(p["SA"][i, k // 32])) *
                           frac_value(int(cb[j, k]), int(p["SB"][j, k // 32]))) for k in range(K))
            assert Fraction(ref[i, j]) == exact        # exact in fp64 at these sizes
            assert Fraction(mag[i, j]) == emag
            assert dref[i, j] == rne_bf16_fraction(exact) or (dref[i, j] | rne_bf16_fraction(exact)) & 0x7FFF == 0
            mant, ex, as_d, as_h = oracle.dot_exact(p["A"], p["SA"], p["B"], p["SB"], K, i, j)
            assert Fraction(mant) * Fraction(2) ** ex == exact
            assert as_h == rne_bf16_fraction(exact) or (as_h | rne_bf16_fraction(exact)) & 0x7FFF == 0


def test_all_code_pairs_single_block():
    """Every (code_a, code_b) pair and a spread of scale pairs, K = 32."""
    K = 32
    for sa, sb in [(127, 127), (120, 133), (1, 200), (254, 100)]:
        for ca in range(16):
            A = np.full((1, 16), ca | (ca << 4), dtype=np.uint8)
            # 16 rows of B, row j holding code j in every element
            B = np.array([[cb | (cb << 4)] * 16 for cb in range(16)], dtype=np.uint8)
            SA = np.full((1, 1), sa, dtype=np.uint8)
            SB = np.full((16, 1), sb, dtype=np.uint8)
            ref, _, dref = oracle.mxgemm(A, SA, B, SB, K)
            for cb in range(16):
                exact = 32 * frac_value(ca, sa) * frac_value(cb, sb)
                assert Fraction(ref[0, cb]) == exact, (ca, cb, sa, sb)
                h = rne_bf16_fraction(exact)
                assert dref[0, cb] == h or (dref[0, cb] | h) & 0x7FFF == 0


def test_numpy_matmul_exact_range():
    """With exponents 124..130 every partial sum is a multiple of 2^-8 below
    2^40, so float64 sums are exact in any order: numpy's matmul on
    independently dequantized operands must agree bit for bit."""
    M, N, K = 48, 40, 1024
    p = small_problem(M, N, K, seed=7, e=(124, 130), beta=1.0, c_sigma=1.0)
    p["alpha"], p["beta"] = 1.0, 0.0
    ref, _, _ = _gemm(p)
    A, B = dequant_np(p["A"], p["SA"], K), dequant_np(p["B"], p["SB"], K)
    assert np.array_equal(ref, A @ B.T)


def test_numpy_matmul_wide_range_close():
    M, N, K = 16, 24, 2048
    p = small_problem(M, N, K, seed=8, e=(110, 140), dist="half_zero")
    ref, mag, _ = _gemm(p)
    A, B = dequant_np(p["A"], p["SA"], K), dequant_np(p["B"], p["SB"], K)
    assert np.all(np.abs(ref - A @ B.T) <= 1e-13 * mag + 1e-300)
    assert np.allclose(mag, np.abs(A) @ np.abs(B).T, rtol=1e-14, atol=0)


def test_exact_mode_agrees_with_fp64_on_wide_exponents():
    # skinny-deep style draws: the fp64 sum may round; it must equal the exact
    # sum rounded once, within a few ulps of the magnitude sum
    M, N, K = 2, 3, 16384
    p = small_problem(M, N, K, seed=9, e=(110, 140), dist="half_zero")
    ref, mag, dref = _gemm(p)
    for i in range(M):
        for j in range(N):
            mant, ex, as_d, as_h = oracle.dot_exact(p["A"], p["SA"], p["B"], p["SB"], K, i, j)
            assert abs(ref[i, j] - as_d) <= 2.0 ** -50 * mag[i, j]
            assert dref[i, j] == as_h or abs(oracle.bf16_to_float(dref[i, j]) - oracle.bf16_to_float(as_h)) \
                <= 2.0 ** -7 * abs(as_d)


def test_alpha_beta_linearity():
    M, N, K = 16, 32, 256
    p = small_problem(M, N, K, seed=21, beta=1.0, c_sigma=1.0)
    p["alpha"], p["beta"] = 1.0, 0.0
    P, _, _ = _gemm(p)
    Cv = np.vectorize(oracle.bf16_to_float)(p["C"])
    for a, b in [(0.5, 1.0), (2.0 ** 5, -0.25), (-3.0, 2.0)]:
        p["alpha"], p["beta"] = a, b
        r, _, _ = _gemm(p)
        assert np.allclose(r, a * P + b * Cv, rtol=1e-15, atol=1e-300)
    # alpha = 2^p scales exactly
    p["alpha"], p["beta"] = 2.0 ** -3, 0.0
    r, _, _ = _gemm(p)
    assert np.array_equal(r, P * 2.0 ** -3)


def test_zero_A_gives_bf16_of_beta_C():
    M, N, K = 8, 16, 64
    p = small_problem(M, N, K, seed=22, beta=1.0, c_sigma=2.0)
    p["A"][:] = 0
    p["beta"] = 0.75
    r, _, d = _gemm(p)
    Cv = np.vectorize(oracle.bf16_to_float)(p["C"])
    assert np.array_equal(r, 0.75 * Cv)
    expect = np.vectorize(lambda v: rne_bf16_fraction(Fraction(float(v))))(0.75 * Cv)
    assert np.array_equal(d, expect.astype(np.uint16))


def test_f32_C_enters_exactly():
    """An f32 C (the bias type the asm_f4gemm README's "C / bias" note
    names) enters at its full f32 value: with A = 0 the reference is
    beta * C exactly, including values bf16 cannot hold, and the stored D
    is that value rounded once to bf16."""
    M, N, K = 8, 16, 64
    p = small_problem(M, N, K, seed=24)
    p["A"][:] = 0
    rng = np.random.default_rng(25)
    Cf = (rng.standard_normal((M, N)) * 3.0).astype(np.float32)
    Cf[0, 0] = np.float32(1.0 + 2.0 ** -20)  # not a bf16 value
    p["C"], p["beta"] = Cf, -0.5
    r, _, d = _gemm(p)
    assert np.array_equal(r, -0.5 * Cf.astype(np.float64))
    assert r[0, 0] == -0.5 * (1.0 + 2.0 ** -20)
    expect = np.vectorize(lambda v: rne_bf16_fraction(Fraction(float(v))))(r)
    assert np.array_equal(d, expect.astype(np.uint16))


def test_f32_C_holding_bf16_values_matches_bf16_C():
    M, N, K = 16, 24, 256
    p = small_problem(M, N, K, seed=26, beta=1.0, c_sigma=1.0)
    p["beta"] = 0.625
    r16, m16, d16 = _gemm(p)
    p["C"] = np.vectorize(oracle.bf16_to_float)(p["C"]).astype(np.float32)
    r32, m32, d32 = _gemm(p)
    assert np.array_equal(r16, r32) and np.array_equal(m16, m32) and np.array_equal(d16, d32)


def test_beta_zero_ignores_C():
    M, N, K = 4, 8, 64
    p = small_problem(M, N, K, seed=23)
    r0, _, _ = _gemm(p)
    p["C"] = np.full((M, N), 0x7FC0, dtype=np.uint16)  # NaN everywhere
    r1, _, _ = _gemm(p)
    assert np.array_equal(r0, r1)


def test_sign_flip_and_scale_step():
    M, N, K = 8, 8, 128
    p = small_problem(M, N, K, seed=24)
    r0, _, _ = _gemm(p)
    q = dict(p)
    q["A"] = p["A"] ^ 0x88  # flip the sign bit of both nibbles
    r1, _, _ = _gemm(q)
    assert np.array_equal(r1, -r0)
    q = dict(p)
    q["SA"] = p["SA"] + 1   # every A scale doubles
    r2, _, _ = _gemm(q)
    assert np.array_equal(r2, 2 * r0)


def test_transpose_symmetry():
    M, N, K = 12, 20, 256
    p = small_problem(M, N, K, seed=25)
    r, _, _ = _gemm(p)
    q = dict(p, A=p["B"], B=p["A"], SA=p["SB"], SB=p["SA"])
    rt, _, _ = _gemm(q)
    assert np.array_equal(r, rt.T)


def test_block_permutation_invariance():
    """Permuting the 32-element K blocks of both operands (with their scales)
    permutes the terms of an exact sum: same value."""
    M, N, K = 6, 10, 256
    p = small_problem(M, N, K, seed=26, e=(124, 130))
    r, _, _ = _gemm(p)
    perm = np.array([3, 7, 0, 5, 1, 6, 2, 4])
    def permute(X, SX):
        Xb = X.reshape(X.shape[0], K // 32, 16)[:, perm, :].reshape(X.shape[0], K // 2)
        return Xb, SX[:, perm]
    A2, SA2 = permute(p["A"], p["SA"])
    B2, SB2 = permute(p["B"], p["SB"])
    r2, _, _ = _gemm(dict(p, A=A2, SA=SA2, B=B2, SB=SB2))
    assert np.array_equal(r, r2)


def test_scale_applies_to_its_own_block():
    K = 128
    A = np.full((1, K // 2), 0x22, dtype=np.uint8)      # all 1.0
    B = np.full((1, K // 2), 0x22, dtype=np.uint8)
    SA = np.array([[127, 128, 127, 127]], dtype=np.uint8)  # block 1 doubled
    SB = np.array([[127, 127, 126, 127]], dtype=np.uint8)  # block 2 halved
    r, m, _ = oracle.mxgemm(A, SA, B, SB, K)
    assert r[0, 0] == 32 * (1 + 2 + 0.5 + 1)
    assert m[0, 0] == r[0, 0]


def test_strided_operands_match_dense():
    M, N, K = 10, 14, 192
    p = small_problem(M, N, K, seed=27, beta=1.0, c_sigma=1.0)
    p["beta"] = 0.5
    r, m, d = _gemm(p)
    pad = lambda X, extra, fill: np.concatenate(
        [X, np.full((X.shape[0], extra), fill, dtype=X.dtype)], axis=1)
    rs, ms, ds = oracle.mxgemm(pad(p["A"], 16, 0xFF), pad(p["SA"], 3, 0xFF),
                               pad(p["B"], 32, 0x77), pad(p["SB"], 5, 0xFF), K,
                               p["alpha"], 0.5,
                               pad(p["C"], 7, 0x7FC0),
                               lda=K + 32, ldb=K + 64, ldsa=K // 32 + 3, ldsb=K // 32 + 5, ldc=N + 7)
    assert np.array_equal(r, rs) and np.array_equal(m, ms) and np.array_equal(d, ds)


def test_row_column_subsets_match_full():
    M, N, K = 20, 30, 256
    p = small_problem(M, N, K, seed=28)
    r, m, d = _gemm(p)
    rows, cols = np.array([19, 0, 7]), np.array([29, 3, 3, 11])
    rs, ms, ds = _gemm(p, rows=rows, cols=cols)
    assert np.array_equal(rs, r[np.ix_(rows, cols)])
    assert np.array_equal(ds, d[np.ix_(rows, cols)])


def test_nan_scale_gives_nan():
    K = 64
    A = np.full((1, K // 2), 0x11, dtype=np.uint8)
    B = np.full((1, K // 2), 0x11, dtype=np.uint8)
    SA = np.array([[127, 255]], dtype=np.uint8)
    SB = np.array([[127, 127]], dtype=np.uint8)
    r, _, d = oracle.mxgemm(A, SA, B, SB, K)
    assert math.isnan(r[0, 0]) and (d[0, 0] & 0x7FFF) > 0x7F80


def test_workload_generators_are_deterministic_and_in_range():
    p1 = inputs.make_problem(16, 32, 256, seed=5, dist="half_zero", e=(110, 140), beta=1.0, c_sigma=2.0)
    p2 = inputs.make_problem(16, 32, 256, seed=5, dist="half_zero", e=(110, 140), beta=1.0, c_sigma=2.0)
    for k in ("A", "B", "SA", "SB", "C"):
        assert np.array_equal(p1[k], p2[k])
    assert p1["SA"].min() >= 110 and p1["SA"].max() <= 140
    codes = unpack_codes_np(p1["B"], 256)
    frac0 = (codes == 0).mean()
    assert 0.4 < frac0 < 0.6
    u = inputs.make_problem(64, 64, 1024, seed=6)
    cu = np.bincount(unpack_codes_np(u["A"], 1024).ravel(), minlength=16)
    assert cu.min() > 0.8 * cu.mean()

"""CPU pins of the oracle's MN-major B layout (b_layout=1).

"CDNA4 MFMA transpose load builtins" (opening section) lets an operand sit
MN-major, B as row-major [K][N]: row k holds the N columns' codes at that k,
packed two per byte like the K-major rows of "Data layouts" (element j of a
row in the low nibble of byte j/2 when j is even).  The scales stay one per
column and 32-block of k, [N][K/32].  These tests tie that reading to values
fixed independently of the oracle's MN-major branch:
  - a permutation matrix: column n of B selects row pi(n) of A^T, so D's
    column n is A's column pi(n) exactly (a swapped n/k role selects
    pi^-1 instead);
  - a nibble-level transpose (written here with plain numpy indexing) of a
    K-major B gives bit-identical results through the oracle's pinned
    K-major branch, for ragged N and padded row pitches;
  - exact rational sums read straight from the MN-major bytes.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from test_oracle import dequant_np, frac_value, rne_bf16_fraction, small_problem, unpack_codes_np


def to_kn(B_nk: np.ndarray, N: int, K: int, ldb: int) -> np.ndarray:
    """K-major [N][K/2] bytes -> MN-major [K][ldb/2] bytes (pad nibbles 0)."""
    codes = unpack_codes_np(B_nk, K)  # [N][K]
    kn = np.zeros((K, ldb), dtype=np.uint8)
    kn[:, :N] = codes.T
    return (kn[:, 0::2] | (kn[:, 1::2] << 4)).astype(np.uint8)


def test_input_helper_is_the_same_transpose():
    """inputs.to_mn_major (used by the GPU tests) moves the codes exactly as
    the transpose above does."""
    from block_scaled_precision_mxfp4_amd import inputs
    p = small_problem(4, 37, 96, seed=9)
    assert np.array_equal(inputs.to_mn_major(p["B"], 37, 96, 64), to_kn(p["B"], 37, 96, 64))
    kn = inputs.to_mn_major(p["B"], 37, 96, 64, pad=7)
    assert (kn[:, 19:] == 0x77).all() and (kn[:, 18] >> 4 == 7).all()


def kn_code(B_kn: np.ndarray, k: int, n: int) -> int:
    byte = int(B_kn[k, n // 2])
    return (byte >> 4) if (n & 1) else (byte & 0xF)


def test_permutation_matrix_selects_columns_of_A():
    M, N, K = 64, 96, 256
    p = small_problem(M, N, K, seed=0x4B4E, e=(120, 134))
    rng = np.random.default_rng(5)
    pi = rng.permutation(K)[:N]
    B_kn = np.zeros((K, N // 2), dtype=np.uint8)
    for n in range(N):
        B_kn[pi[n], n // 2] |= (0x2 << 4) if (n & 1) else 0x2  # 1.0
    SB = np.full((N, K // 32), 127, dtype=np.uint8)
    ref, mag, dref = oracle.mxgemm(p["A"], p["SA"], B_kn, SB, K, b_layout=1, ldb=N)
    A = dequant_np(p["A"], p["SA"], K)
    assert np.array_equal(ref, A[:, pi])
    assert np.array_equal(mag, np.abs(A[:, pi]))
    expect = np.array([[rne_bf16_fraction(Fraction(float(v))) for v in row] for row in A[:, pi]], dtype=np.uint16)
    assert (((dref == expect) | (((dref | expect) & 0x7FFF) == 0))).all()


@pytest.mark.parametrize("M,N,K,pad", [(16, 64, 512, 0), (33, 37, 288, 1), (7, 130, 1024, 30), (1, 256, 4096, 0)])
def test_matches_k_major_on_a_transposed_copy(M, N, K, pad):
    p = small_problem(M, N, K, seed=0x7A + N, e=(112, 140), beta=1.0, c_sigma=1.0)
    ldb = N + (N & 1) + pad * 2
    B_kn = to_kn(p["B"], N, K, ldb)
    a = oracle.mxgemm(p["A"], p["SA"], p["B"], p["SB"], K, 0.75, -0.5, p["C"])
    b = oracle.mxgemm(p["A"], p["SA"], B_kn, p["SB"], K, 0.75, -0.5, p["C"], b_layout=1, ldb=ldb)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_exact_sums_from_mn_major_bytes():
    M, N, K = 3, 5, 96
    p = small_problem(M, N, K, seed=0x3E, e=(120, 134))  # fp64 sums exact
    B_kn = to_kn(p["B"], N, K, 6)
    ref, _, dref = oracle.mxgemm(p["A"], p["SA"], B_kn, p["SB"], K, b_layout=1, ldb=6)
    ca = unpack_codes_np(p["A"], K)
    for i in range(M):
        for j in range(N):
            s = sum(frac_value(int(ca[i, k]), int(p["SA"][i, k // 32])) *
                    frac_value(kn_code(B_kn, k, j), int(p["SB"][j, k // 32])) for k in range(K))
            assert Fraction(ref[i, j]) == s
            assert dref[i, j] == rne_bf16_fraction(s)

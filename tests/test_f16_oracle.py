"""Pins for the oracle's FP16 GEMM (the "FP16 GEMM example" of "CDNA4 MFMA
transpose load builtins": fp32 C = fp16 A [M, K] x fp16 B [K, N], B
K-major).  Each expectation is independent of the oracle's code: numpy's
float16 for the element decoding, numpy's fp64 matrix product on small
exactly-summable inputs, the identity and the transpose."""
import numpy as np

import oracle
from block_scaled_precision_mxfp4_amd import inputs


def test_f16_decoding_matches_numpy_on_every_code():
    codes = np.arange(1 << 16, dtype=np.uint16)
    want = codes.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_float(int(c)) for c in codes])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_gemm_matches_numpy_fp64_product():
    rng = np.random.default_rng(5)
    M, N, K = 7, 24, 40
    # integers and halves below 2^6: every partial sum is exact in fp64
    A = (rng.integers(-64, 64, (M, K)) / 2.0).astype(np.float16)
    B = (rng.integers(-64, 64, (K, N)) / 2.0).astype(np.float16)
    ref, mag = oracle.f16_gemm(A.view(np.uint16), B.view(np.uint16), K)
    want = A.astype(np.float64) @ B.astype(np.float64)
    assert np.array_equal(ref, want)
    assert np.array_equal(mag, np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64)))


def test_identity_and_transpose():
    M, K = 9, 16
    A = inputs.gaussian_f16(0x16, M, K, 2.0)
    eye = np.eye(K, dtype=np.float16).view(np.uint16)
    ref, _ = oracle.f16_gemm(A, eye, K)
    assert np.array_equal(ref, A.view(np.float16).astype(np.float64))
    B = inputs.gaussian_f16(0x17, K, 8, 1.0)
    ab, _ = oracle.f16_gemm(A, B, K)
    bt_at, _ = oracle.f16_gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), K)
    assert np.allclose(ab, bt_at.T, rtol=1e-14, atol=1e-300)


def test_strides_and_subsets():
    M, N, K = 5, 16, 24
    A = inputs.gaussian_f16(0x18, M, K, 1.0)
    B = inputs.gaussian_f16(0x19, K, N, 1.0)
    full, _ = oracle.f16_gemm(A, B, K)
    Ap = np.zeros((M, K + 8), dtype=np.uint16)
    Ap[:, :K] = A
    Bp = np.full((K, N + 16), 0x7E00, dtype=np.uint16)  # NaN padding must not be read
    Bp[:, :N] = B
    pad, _ = oracle.f16_gemm(Ap, Bp, K, lda=K + 8, ldb=N + 16, cols=np.arange(N))
    assert np.array_equal(full, pad)
    sub, _ = oracle.f16_gemm(A, B, K, rows=[4, 0], cols=[15, 3])
    assert np.array_equal(sub, full[np.ix_([4, 0], [15, 3])])

"""GPU parity of mxgemm_f16_run (fp32 C = fp16 A x K-major fp16 B, B read
from LDS with the 16-bit transpose loads) against the oracle, through the
C-ABI.

Bound per element: |C - ref| <= K * 2^-24 * mag + 2^-24 * |ref|, mag =
sum_k |a_ik b_kj|: fp16 products are exact in fp32, and any order of fp32
additions of K terms errs by at most (K - 1) units of 2^-24 relative to the
sum of magnitudes, plus the final value's own rounding.  Cases cover one
tile, several tiles with ragged M/N/K edges, M = 1, padded strides, and
the 8192^3 shape on sampled rows.
"""
import sys

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
import oracle
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def f16_gpu(A, B, M, N, K, lda=None, ldb=None, ldc=None):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    Ap = np.zeros((M, lda), dtype=np.uint16)
    Ap[:, :A.shape[1]] = A
    Bp = np.full((K, ldb), 0x7E00, dtype=np.uint16)  # NaN padding: must never be read
    Bp[:, :B.shape[1]] = B
    Ad = torch.from_numpy(Ap.view(np.int16)).cuda()
    Bd = torch.from_numpy(Bp.view(np.int16)).cuda()
    C = torch.full((M, ldc), float("nan"), dtype=torch.float32, device="cuda")
    mx.mxgemm_f16_run(C, Ad, Bd, M, N, K, lda=lda, ldb=ldb, ldc=ldc)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def check(C, ref, mag, K, what):
    err = np.abs(C.astype(np.float64) - ref)
    bound = K * 2.0 ** -24 * mag + 2.0 ** -24 * np.abs(ref)
    bad = ~(err <= bound)
    assert not bad.any(), "%s: %d of %d outside the bound (worst %.3g)" % (
        what, int(bad.sum()), bad.size, float((err - bound).max()))


CASES = [(256, 256, 512), (300, 520, 1000), (1, 8, 8), (17, 264, 72), (512, 1024, 2048), (257, 264, 4104)]


@pytest.mark.parametrize("shape", CASES, ids=lambda s: "%dx%dx%d" % s)
def test_f16_matches_oracle(shape):
    M, N, K = shape
    A = inputs.gaussian_f16(0xF16 + M, M, K, 1.0)
    B = inputs.gaussian_f16(0xF17 + N, K, N, 1.0)
    say("case f16", shape)
    C = f16_gpu(A, B, M, N, K)
    ref, mag = oracle.f16_gemm(A, B, K)
    check(C, ref, mag, K, "f16 %s" % (shape,))


def test_f16_padded_strides_leave_padding():
    M, N, K = 130, 136, 200
    lda, ldb, ldc = K + 24, N + 40, N + 8
    A = inputs.gaussian_f16(0xF18, M, K, 1.0)
    B = inputs.gaussian_f16(0xF19, K, N, 1.0)
    C = f16_gpu(A, B, M, N, K, lda=lda, ldb=ldb, ldc=ldc)
    ref, mag = oracle.f16_gemm(A, B, K)
    check(C[:, :N], ref, mag, K, "f16 strided")
    assert np.isnan(C[:, N:]).all(), "C padding was written"


def test_f16_square_8192_sampled():
    M = N = K = 8192
    A = inputs.gaussian_f16(0xF1A, M, K, 1.0)
    B = inputs.gaussian_f16(0xF1B, K, N, 1.0)
    say("case f16 8192^3")
    C = f16_gpu(A, B, M, N, K)
    rng = np.random.default_rng(16)
    rows = np.sort(np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 14)])))
    cols = np.sort(np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 1022)])))
    ref, mag = oracle.f16_gemm(A, B, K, rows=rows, cols=cols)
    check(C[np.ix_(rows, cols)], ref, mag, K, "f16 8192^3 sample")

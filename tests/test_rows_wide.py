"""GPU parity of the rows kernel (16 < M <= 64) with A in a wider format:
FP8 E4M3, BF8 E5M2, FP6 E2M3 or FP6 E3M2 against FP4 B (the scaled matrix
instruction's mixed inputs, "CDNA4 dense MFMA builtins", "Mixed-precision
with scaling"), through the C-ABI, against the oracle's exact fp64 reference
with the per-element tolerance of the FP4 tests.

A is staged in LDS per batch of four 128-K steps: the 8-bit rows as 32
16-byte chunks, dense FP6 rows (24 bytes per K-block) as 24 chunks, each
K-block's operand then read as two 16-byte or three 8-byte pieces.  Cases
cover every 16-row group count (2, 3, 4), ragged M and N, chunks that end
inside a batch, split K, packed and row-major B, padded rows with an 8-byte
FP6 pitch, scale rows at odd pitches and addresses (per-wave scale loads),
and an FP6 K-block count that is odd (planned on the 8-bit tiles instead).
"""
import sys

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxgpu import assert_parity, dev_bf16, dev_u8, gemm_gpu, host_bits, oracle_ref  # noqa: E402

FORMATS = [mx.FMT_FP8_E4M3, mx.FMT_FP8_E5M2, mx.FMT_FP6_E2M3, mx.FMT_FP6_E3M2]
NAMES = {1: "e4m3", 2: "e5m2", 3: "e2m3", 4: "e3m2"}
PREFIX = {1: "rows_fp8", 2: "rows_bf8", 3: "rows_fp6", 4: "rows_fp6"}
BITS = {1: 8, 2: 8, 3: 6, 4: 6}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def problem(M, N, K, fmt, seed, c=True):
    # FP8 products stay inside fp32's range with these scale exponents
    e = (120, 134) if fmt in (3, 4) else (112, 130)
    p = inputs.make_problem(M, N, K, seed=seed, e=e, beta=1.0 if c else 0.0, c_sigma=1.0 if c else None, a_fmt=fmt)
    p["alpha"], p["beta"] = (1.5, -0.75) if c else (0.5, 0.0)
    return p


def plan_name(M, N, K, fmt, split=-1, packed=0):
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, b_packed=packed, a_format=fmt)
    return mx.mxgemm_plan_ex(M, N, K, st, split, 256)["kernel_name"]


ROWS_CASES = [(17, 200, 2048), (40, 1000, 1024), (64, 333, 4096), (50, 4096, 8192), (33, 64, 512),
              (48, 520, 1088)]


@pytest.mark.parametrize("fmt", FORMATS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("shape", ROWS_CASES, ids=lambda s: "%dx%dx%d" % s)
def test_rows_wide_matches_oracle(shape, fmt):
    """Row-major and packed B, unsplit and split K (the split results are
    deterministic: a repeated call gives the same bits)."""
    M, N, K = shape
    p = problem(M, N, K, fmt, seed=0x3077 + 31 * fmt + M + N)
    ref, mag, _ = oracle_ref(p)
    assert plan_name(M, N, K, fmt, 1).startswith(PREFIX[fmt] + "_m%dx16" % -(-M // 16))
    for packed in (False, True):
        for s in (1, 2, 4):
            say("case rows wide", NAMES[fmt], shape, "packed", packed, "split", s)
            d = gemm_gpu(p, split_k=s, b_packed=packed)
            assert_parity(d, ref, mag, "rows %s %s packed=%s split=%d" % (NAMES[fmt], shape, packed, s))
            if s == 4:
                assert np.array_equal(gemm_gpu(p, split_k=4, b_packed=packed), d)


@pytest.mark.parametrize("fmt", FORMATS, ids=lambda f: NAMES[f])
def test_rows_wide_strided(fmt):
    """Padded A and B rows (FP6: a byte pitch that is a multiple of 8 but not
    of 16), scale pitches that are not multiples of 16 and scales at odd
    addresses (the per-wave scale loads), padded C and D."""
    M, N, K = 44, 301, 2048
    p = problem(M, N, K, fmt, seed=0x5717 + fmt)
    ref, mag, _ = oracle_ref(p)
    lda, ldb, ldsa, ldsb, ldc, ldd = K + 32, K + 96, K // 32 + 3, K // 32 + 5, N + 3, N + 1
    a_row = lda * BITS[fmt] // 8
    if fmt in (3, 4):
        assert a_row % 8 == 0 and a_row % 16 != 0

    def pad(X, cols, fill):
        out = np.full((X.shape[0], cols), fill, dtype=X.dtype)
        out[:, : X.shape[1]] = X
        return out
    A = dev_u8(pad(p["A"], a_row, 0x55))
    B = dev_u8(pad(p["B"], ldb // 2, 0x77))
    SA_buf = dev_u8(np.concatenate([[0xFF], pad(p["SA"], ldsa, 0xFF).ravel()]))
    SB_buf = dev_u8(np.concatenate([[0xFF], pad(p["SB"], ldsb, 0xFF).ravel()]))
    C = dev_bf16(pad(p["C"], ldc, 0x7FC0))
    D = torch.zeros((M, ldd), dtype=torch.bfloat16, device="cuda")
    st = mx.make_strides(ldd=ldd, ldc=ldc, lda=lda, ldb=ldb, ldsa=ldsa, ldsb=ldsb, a_format=fmt)
    assert mx.mxgemm_plan_ex(M, N, K, st, 1, 256)["kernel_name"].startswith(PREFIX[fmt])
    for s in (1, 4):
        say("case rows wide strided", NAMES[fmt], "split", s)
        mx.mxgemm_run(D, C, A, B, SA_buf.data_ptr() + 1, SB_buf.data_ptr() + 1, p["alpha"], p["beta"], M, N, K,
                      strides=st, split_k=s)
        torch.cuda.synchronize()
        d = host_bits(D)
        assert_parity(d[:, :N], ref, mag, "rows wide strided %s split %d" % (NAMES[fmt], s))
        assert (d[:, N:] == 0).all()  # padding columns untouched


@pytest.mark.parametrize("fmt", [mx.FMT_FP6_E2M3, mx.FMT_FP6_E3M2], ids=lambda f: NAMES[f])
def test_fp6_odd_block_count_takes_the_8bit_tiles(fmt):
    """K = 1056 (33 K-blocks): a 16-byte chunk of a dense FP6 row would
    straddle the end of K, so the plan is the 8-bit tiles on the re-laid
    copy of A."""
    M, N, K = 40, 300, 1056
    assert plan_name(M, N, K, fmt).startswith("tile_a8")
    p = problem(M, N, K, fmt, seed=0x0DD + fmt)
    ref, mag, _ = oracle_ref(p)
    say("case fp6 odd blocks", NAMES[fmt])
    assert_parity(gemm_gpu(p), ref, mag, "fp6 odd K-blocks %s" % NAMES[fmt])


@pytest.mark.parametrize("fmt", FORMATS, ids=lambda f: NAMES[f])
def test_rows_wide_prefill_shape_sampled(fmt):
    """64 x 7168 x 16384 (the small-batch workload's shape) in the planned
    launch, on 40 sampled columns of every row, first and last included."""
    M, N, K = 64, 7168, 16384
    p = problem(M, N, K, fmt, seed=0x64 + fmt, c=False)
    rng = np.random.default_rng(fmt)
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 38, replace=False)]))
    say("case rows wide 64x7168x16384", NAMES[fmt], plan_name(M, N, K, fmt))
    d = gemm_gpu(p)
    ref, mag, _ = oracle_ref(p, cols=cols)
    assert_parity(d[:, cols], ref, mag, "rows wide 64x7168x16384 %s" % NAMES[fmt])

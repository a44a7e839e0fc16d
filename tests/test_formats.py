"""GPU parity of mixed-format GEMMs, through the C-ABI: A in FP8 E4M3,
BF8 E5M2, FP6 E2M3 or FP6 E3M2 (the other inputs of the scaled matrix
instructions, "CDNA4 dense MFMA builtins", "Mixed-precision with scaling"),
B in FP4, against the oracle's exact fp64 reference with the per-element
tolerance of the FP4 tests.

Cases cover the single-row path (M = 1), one 16-row block, several blocks
with a ragged last one, K tails, ragged N, forced split-K, packed B, and C
in bf16 and f32; the 1 x 8192 x 8192 decode shape is checked on sampled
columns.
"""
import sys

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxgpu import assert_parity, gemm_gpu, oracle_ref  # noqa: E402

FORMATS = [mx.FMT_FP8_E4M3, mx.FMT_FP8_E5M2, mx.FMT_FP6_E2M3, mx.FMT_FP6_E3M2]
NAMES = {1: "e4m3", 2: "e5m2", 3: "e2m3", 4: "e3m2"}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# (M, N, K, split, b_packed, C): C None, "bf16" or "f32"
CASES = [
    (1, 1000, 2048, 1, False, None),
    (1, 777, 1056, -1, False, "bf16"),
    (5, 512, 4096, 4, False, None),
    (16, 300, 512, 1, True, "f32"),
    (17, 640, 2048, 2, False, "bf16"),
    (40, 333, 1024, 1, True, None),
    (70, 256, 4096, 8, False, "f32"),
]


def problem(case, fmt, seed):
    M, N, K, split, packed, c = case
    e = (120, 134) if fmt in (3, 4) else (110, 130)  # keep FP8 products inside fp32's range
    p = inputs.make_problem(M, N, K, seed=seed, e=e, beta=0.0 if c is None else 1.0,
                            c_sigma=None if c is None else 2.0, a_fmt=fmt)
    if c == "f32":
        rng = np.random.default_rng(seed)
        p["C"] = (rng.standard_normal((M, N)) * 2.0).astype(np.float32)
    if c is not None:
        p["beta"] = -0.75
    p["alpha"] = 0.5
    return p


@pytest.mark.parametrize("fmt", FORMATS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%dx%d_s%d%s%s" % (
    c[0], c[1], c[2], c[3], "_packed" if c[4] else "", "_" + c[5] if c[5] else ""))
def test_mixed_format_matches_oracle(case, fmt):
    M, N, K, split, packed, c = case
    p = problem(case, fmt, seed=0xF0F0 + 97 * fmt + M * 7 + N)
    say("case", NAMES[fmt], case)
    d = gemm_gpu(p, split_k=split, b_packed=packed)
    ref, mag, _ = oracle_ref(p)
    assert_parity(d, ref, mag, "%s %s" % (NAMES[fmt], case))


@pytest.mark.parametrize("fmt", FORMATS, ids=lambda f: NAMES[f])
def test_decode_shape_sampled(fmt):
    """1 x 8192 x 8192, the decode shape of the M = 1 workload, with A in
    the wider format; 256 sampled columns against the oracle."""
    M = 1
    N = K = 8192
    p = inputs.make_problem(M, N, K, seed=0xDEC + fmt, e=(120, 134) if fmt in (3, 4) else (115, 128),
                            a_fmt=fmt)
    p["alpha"] = 0.5
    say("case decode", NAMES[fmt])
    d = gemm_gpu(p)
    cols = np.sort(np.random.default_rng(fmt).choice(N, 256, replace=False))
    ref, mag, _ = oracle_ref(p, cols=cols)
    assert_parity(d[:, cols], ref, mag, "decode %s" % NAMES[fmt])



# 8-bit A with M > 16 runs on the tiled kernel with 8-bit A tiles
CASES_A8 = [
    (300, 520, 1056, -1, False, "bf16"),  # K tail (blocks past a stage's end)
    (512, 1024, 2048, 1, True, None),     # packed B
    (256, 768, 4096, 4, False, "f32"),    # forced split, f32 C
    (129, 96, 512, 1, False, None),       # ragged M and N
]


@pytest.mark.parametrize("fmt", [mx.FMT_FP8_E4M3, mx.FMT_FP8_E5M2], ids=lambda f: NAMES[f])
@pytest.mark.parametrize("case", CASES_A8, ids=lambda c: "%dx%dx%d_s%d%s%s" % (
    c[0], c[1], c[2], c[3], "_packed" if c[4] else "", "_" + c[5] if c[5] else ""))
def test_fp8_tiled_matches_oracle(case, fmt):
    M, N, K, split, packed, c = case
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, b_packed=int(packed), a_format=fmt)
    assert mx.mxgemm_plan_ex(M, N, K, st, split, 256)["kernel"] == 3
    p = problem(case, fmt, seed=0xA8A8 + 31 * fmt + M + N)
    say("case tiled", NAMES[fmt], case)
    d = gemm_gpu(p, split_k=split, b_packed=packed)
    ref, mag, _ = oracle_ref(p)
    assert_parity(d, ref, mag, "tiled %s %s" % (NAMES[fmt], case))


def test_fp8_tiled_large_sampled():
    M, N, K = 2048, 2048, 4096
    fmt = mx.FMT_FP8_E4M3
    p = inputs.make_problem(M, N, K, seed=0xA8A9, e=(115, 128), a_fmt=fmt)
    say("case tiled 2048x2048x4096")
    d = gemm_gpu(p, b_packed=True)
    rng = np.random.default_rng(8)
    rows = np.sort(rng.choice(M, 24, replace=False))
    ref, mag, _ = oracle_ref(p, rows=rows)
    assert_parity(d[rows], ref, mag, "tiled 2048x2048x4096")


# FP6 A with M > 16: A re-laid into 32-byte blocks (codes unchanged), then the
# tiled kernel's 8-bit A tiles with the FP6 operand format
@pytest.mark.parametrize("fmt", [mx.FMT_FP6_E2M3, mx.FMT_FP6_E3M2], ids=lambda f: NAMES[f])
@pytest.mark.parametrize("M,kernel", [(32, 2), (80, 3)], ids=["rows", "tiles"])
def test_fp6_all_codes_through_the_wide_kernels(fmt, M, kernel):
    """B = I (FP4 1.0 on the diagonal, unit scales): D is A dequantized, and
    every FP6 value has at most 4 significant bits, so D must equal the
    oracle's bf16 result bit for bit.  The rows hold all 64 codes, each row
    a different rotation, with varied scales: 32 rows on the rows kernel
    (dense FP6 staged in LDS), 80 on the 8-bit tiles (re-laid FP6)."""
    K = 64
    N = K
    codes = np.array([[(r + k) % 64 for k in range(K)] for r in range(M)], dtype=np.uint64)
    A = np.zeros((M, K * 6 // 8), dtype=np.uint8)
    for r in range(M):
        acc = 0
        for k in range(K):
            acc |= int(codes[r, k]) << (6 * k)
        A[r] = np.frombuffer(acc.to_bytes(K * 6 // 8, "little"), dtype=np.uint8)
    rng = np.random.default_rng(fmt)
    SA = rng.integers(118, 136, (M, K // 32)).astype(np.uint8)
    B = np.zeros((N, K // 2), dtype=np.uint8)
    for j in range(N):
        B[j, j // 2] |= 0x2 << (4 * (j % 2))
    SB = np.full((N, K // 32), 127, dtype=np.uint8)
    p = dict(M=M, N=N, K=K, A=A, SA=SA, B=B, SB=SB, alpha=1.0, beta=0.0, C=None, a_fmt=fmt)
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, a_format=fmt)
    assert mx.mxgemm_plan_ex(M, N, K, st, -1, 256)["kernel"] == kernel
    say("case fp6 identity", NAMES[fmt], M)
    d = gemm_gpu(p)
    _, _, dref = oracle_ref(p)
    same = (d == dref) | (((d | dref) & 0x7FFF) == 0)  # +0 and -0 are equal
    assert same.all(), "%d of %d elements differ" % (int((~same).sum()), d.size)


FP6_TILED = [
    (300, 520, 1056, -1, False, "bf16"),  # K tail (one block past 128), C
    (40, 96, 608, -1, False, None),       # small tile, K tail of three blocks
    (130, 256, 2080, 2, False, "f32"),    # split-K, f32 C, K tail
    (2048, 2048, 4096, 1, True, None),    # packed B, sampled
]


@pytest.mark.parametrize("fmt", [mx.FMT_FP6_E2M3, mx.FMT_FP6_E3M2], ids=lambda f: NAMES[f])
@pytest.mark.parametrize("case", FP6_TILED, ids=lambda c: "%dx%dx%d" % c[:3])
def test_fp6_tiled_matches_oracle(case, fmt):
    M, N, K, split, packed, c = case
    p = problem(case, fmt, seed=0xF6F6 + 13 * fmt + M)
    say("case fp6 tiled", NAMES[fmt], case)
    d = gemm_gpu(p, split_k=split, b_packed=packed)
    if M * N <= 300 * 520:
        ref, mag, _ = oracle_ref(p)
        assert_parity(d, ref, mag, "fp6 tiled %s %s" % (NAMES[fmt], case))
    else:
        rng = np.random.default_rng(M + fmt)
        rows = np.sort(rng.choice(M, 20, replace=False))
        ref, mag, _ = oracle_ref(p, rows=rows)
        assert_parity(d[rows], ref, mag, "fp6 tiled %s %s" % (NAMES[fmt], case))


# FP6 A on the 256 x 256 dense FP6 tile: A re-laid into the instruction's
# operand order (24 bytes per lane and K-block), A scales shuffled, a
# row-major B packed by the library; forced through the planner's test hook
# on shapes the oracle checks in full
FP6_DENSE = [
    (300, 520, 1056, -1, True, "bf16"),  # ragged M and N, K tail (33 blocks), C
    (300, 520, 1056, -1, False, None),   # the same with row-major B
    (512, 512, 2048, 1, True, None),     # whole tiles, staged epilogue
    (130, 256, 2080, 2, True, "f32"),    # split-K with a K tail, f32 C
    (256, 300, 8192, 4, False, None),    # split-K over whole stages, row-major B
]


@pytest.mark.parametrize("fmt", [mx.FMT_FP6_E2M3, mx.FMT_FP6_E3M2], ids=lambda f: NAMES[f])
@pytest.mark.parametrize("case", FP6_DENSE, ids=lambda c: "%dx%dx%d_s%d%s" % (c[:4] + ("_packed" if c[4] else "",)))
def test_fp6_dense_tile_matches_oracle(case, fmt, monkeypatch):
    """Against the oracle, and bit for bit against the 128 x 256 8-bit tile
    on the padded copy of A: both feed each accumulator the same operands in
    the same K order."""
    M, N, K, split, packed, c = case
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, b_packed=int(packed), a_format=fmt)
    p = problem(case, fmt, seed=0xD6D6 + 13 * fmt + M + N)
    monkeypatch.setenv("MXGEMM_A8_TILE", "tile_fp6_256x256")
    assert mx.mxgemm_plan_ex(M, N, K, st, split, 256)["kernel_name"] == "tile_fp6_256x256"
    say("case fp6 dense", NAMES[fmt], case)
    d = gemm_gpu(p, split_k=split, b_packed=packed)
    ref, mag, _ = oracle_ref(p)
    assert_parity(d, ref, mag, "fp6 dense %s %s" % (NAMES[fmt], case))
    monkeypatch.setenv("MXGEMM_A8_TILE", "tile_a8_128x256")
    assert mx.mxgemm_plan_ex(M, N, K, st, split, 256)["kernel_name"] == "tile_a8_128x256"
    assert np.array_equal(gemm_gpu(p, split_k=split, b_packed=packed), d)


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor_b", "packed_b"])
def test_fp6_dense_tile_strided(packed, monkeypatch):
    """Padded A rows (a byte pitch that is a multiple of 8, not of 16: the
    re-layout's 8-byte reads; and one that is a multiple of 16), padded B
    rows and scale rows at odd pitches and addresses, padded C and D, on the
    dense FP6 tile."""
    from mxgpu import dev_bf16, dev_u8, host_bits
    fmt = mx.FMT_FP6_E2M3
    M, N, K = 272, 300, 2048
    p = problem((M, N, K, 1, packed, "bf16"), fmt, seed=0x57D6 + int(packed))
    ref, mag, _ = oracle_ref(p)
    monkeypatch.setenv("MXGEMM_A8_TILE", "tile_fp6_256x256")
    for lda in (K + 32, K + 64):
        a_row = lda * 6 // 8
        ldb, ldsa, ldsb, ldc, ldd = K + 96, K // 32 + 3, K // 32 + 5, N + 3, N + 1

        def pad(X, cols, fill):
            out = np.full((X.shape[0], cols), fill, dtype=X.dtype)
            out[:, : X.shape[1]] = X
            return out
        A = dev_u8(pad(p["A"], a_row, 0x55))
        SA_buf = dev_u8(np.concatenate([[0xFF], pad(p["SA"], ldsa, 0xFF).ravel()]))
        C = dev_bf16(pad(p["C"], ldc, 0x7FC0))
        D = torch.zeros((M, ldd), dtype=torch.bfloat16, device="cuda")
        if packed:
            info = mx.mxgemm_plan(M, N, K, 1, -1, 256)
            B = torch.empty(info["packed_b_bytes"], dtype=torch.uint8, device="cuda")
            SBp = torch.empty(info["packed_sb_bytes"], dtype=torch.uint8, device="cuda")
            mx.mxgemm_pack_b(B, SBp, dev_u8(p["B"]), dev_u8(p["SB"]), N, K)
            sb_ptr, ldb_e, ldsb_e = SBp.data_ptr(), K, K // 32
        else:
            B = dev_u8(pad(p["B"], ldb // 2, 0x77))
            SB_buf = dev_u8(np.concatenate([[0xFF], pad(p["SB"], ldsb, 0xFF).ravel()]))
            sb_ptr, ldb_e, ldsb_e = SB_buf.data_ptr() + 1, ldb, ldsb
        st = mx.make_strides(ldd=ldd, ldc=ldc, lda=lda, ldb=ldb_e, ldsa=ldsa, ldsb=ldsb_e, b_packed=int(packed),
                             a_format=fmt)
        assert mx.mxgemm_plan_ex(M, N, K, st, 1, 256)["kernel_name"] == "tile_fp6_256x256"
        say("case fp6 dense strided", "lda", lda, "packed", packed)
        mx.mxgemm_run(D, C, A, B, SA_buf.data_ptr() + 1, sb_ptr, p["alpha"], p["beta"], M, N, K, strides=st,
                      split_k=1)
        torch.cuda.synchronize()
        d = host_bits(D)
        assert_parity(d[:, :N], ref, mag, "fp6 dense strided lda %d packed %s" % (lda, packed))
        assert (d[:, N:] == 0).all()  # padding columns untouched


@pytest.mark.parametrize("fmt", [mx.FMT_FP6_E2M3, mx.FMT_FP6_E3M2], ids=lambda f: NAMES[f])
def test_fp6_dense_tile_all_codes(fmt, monkeypatch):
    """B = I through the dense FP6 tile: every FP6 code in every lane
    position of a K-block, D equal to the oracle's bf16 result bit for bit."""
    M, K = 272, 256
    N = K
    codes = np.array([[(3 * r + k) % 64 for k in range(K)] for r in range(M)], dtype=np.uint64)
    A = np.zeros((M, K * 6 // 8), dtype=np.uint8)
    for r in range(M):
        acc = 0
        for k in range(K):
            acc |= int(codes[r, k]) << (6 * k)
        A[r] = np.frombuffer(acc.to_bytes(K * 6 // 8, "little"), dtype=np.uint8)
    rng = np.random.default_rng(16 + fmt)
    SA = rng.integers(118, 136, (M, K // 32)).astype(np.uint8)
    B = np.zeros((N, K // 2), dtype=np.uint8)
    for j in range(N):
        B[j, j // 2] |= 0x2 << (4 * (j % 2))
    SB = np.full((N, K // 32), 127, dtype=np.uint8)
    p = dict(M=M, N=N, K=K, A=A, SA=SA, B=B, SB=SB, alpha=1.0, beta=0.0, C=None, a_fmt=fmt)
    monkeypatch.setenv("MXGEMM_A8_TILE", "tile_fp6_256x256")
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, b_packed=1, a_format=fmt)
    assert mx.mxgemm_plan_ex(M, N, K, st, -1, 256)["kernel_name"] == "tile_fp6_256x256"
    say("case fp6 dense identity", NAMES[fmt])
    d = gemm_gpu(p, b_packed=True)
    _, _, dref = oracle_ref(p)
    same = (d == dref) | (((d | dref) & 0x7FFF) == 0)  # +0 and -0 are equal
    assert same.all(), "%d of %d elements differ" % (int((~same).sum()), d.size)


def test_fp6_conversion_buffers_are_per_stream():
    """FP6 A with M > 16 is re-laid in a buffer owned per (device, stream).  Two problems of different sizes and formats on two streams,
    each launched twice with no synchronization in between, must both match
    the oracle."""
    from mxgpu import dev_u8, host_bits
    cases = [(mx.FMT_FP6_E2M3, 96, 512, 2048), (mx.FMT_FP6_E3M2, 200, 384, 1024)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = []
    for (fmt, M, N, K), s in zip(cases, streams):
        p = inputs.make_problem(M, N, K, seed=0x5757 + fmt, e=(120, 134), a_fmt=fmt)
        p["alpha"] = 0.5
        A, B, SA, SB = dev_u8(p["A"]), dev_u8(p["B"]), dev_u8(p["SA"]), dev_u8(p["SB"])
        D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, a_format=fmt)
        assert mx.mxgemm_plan_ex(M, N, K, st, -1, 256)["kernel"] == 3
        runs.append((p, A, B, SA, SB, D, st, s))
    torch.cuda.synchronize()
    say("case fp6 two streams")
    for _ in range(2):
        for p, A, B, SA, SB, D, st, s in runs:
            mx.mxgemm_run(D, None, A, B, SA, SB, p["alpha"], 0.0, p["M"], p["N"], p["K"], strides=st,
                          stream=s.cuda_stream)
    torch.cuda.synchronize()
    for p, A, B, SA, SB, D, st, s in runs:
        ref, mag, _ = oracle_ref(p)
        assert_parity(host_bits(D), ref, mag, "fp6 stream %d" % p["a_fmt"])

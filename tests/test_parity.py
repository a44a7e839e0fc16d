"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Every test runs libmxgemm's kernels via the Python binding (ctypes into
libmxgemm.so) on seeded synthetic inputs and compares element by element with
the oracle (tolerance in tests/mxgpu.py).  Full-size workloads are compared on
every element where the oracle finishes in seconds, and on a sample of rows
and columns (including first/last tiles) for the 8192^3 case.
"""
import sys

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxgpu import (assert_parity, bf16_to_f64, compare, dev_bf16, dev_u8, gemm_gpu,  # noqa: E402
                   host_bits, oracle_ref)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def lib_loaded():
    # the HIP library must be the one that runs: load it explicitly, no fallback
    mx.lib()
    yield
    mx.mxgemm_release_workspaces()


def _sample_rows_cols(M, N, seed, n=24):
    rng = np.random.default_rng(seed)
    edge_r = [0, 1, 15, 16, 127, 128, 255, 256, M // 2, M - 257, M - 256, M - 1]
    edge_c = [0, 3, 4, 15, 16, 255, 256, 511, N // 2, N - 257, N - 256, N - 1]
    rows = sorted(set([r for r in edge_r if 0 <= r < M] + list(rng.integers(0, M, n))))
    cols = sorted(set([c for c in edge_c if 0 <= c < N] + list(rng.integers(0, N, 3 * n))))
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_parity(name):
    p = inputs.make_workload(name)
    M, N, K = p["M"], p["N"], p["K"]
    say("case", name, "M N K", M, N, K, "packed", p["b_packed"], p["sa_packed"], "seed", hex(p["seed"]))
    d = gemm_gpu(p, split_k=-1, b_packed=p["b_packed"], sa_packed=p["sa_packed"])
    if M * N * K <= 8 * 2 ** 30:
        ref, mag, _ = oracle_ref(p)
        rel = assert_parity(d, ref, mag, name)
    else:
        rows, cols = _sample_rows_cols(M, N, p["seed"])
        ref, mag, _ = oracle_ref(p, rows=rows, cols=cols)
        rel = assert_parity(d[np.ix_(rows, cols)], ref, mag, name)
        assert np.isfinite(bf16_to_f64(d)).all()
    say("  max rel err", rel)


SPLIT_CASES = [
    # (M, N, K, dist, e) : skinny kernel and tiled kernel, with and without K tails
    (1, 8192, 8192, "uniform", (120, 134)),
    (64, 1024, 4096, "half_zero", (110, 140)),
    (512, 1024, 2048, "uniform", (123, 131)),
    (300, 520, 4096, "uniform", (123, 131)),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "%dx%dx%d" % c[:3])
def test_split_k_values_agree_and_are_deterministic(case):
    M, N, K, dist, e = case
    p = inputs.make_problem(M, N, K, seed=0x5EED + M, dist=dist, e=e, beta=1.0, c_sigma=1.0)
    p["alpha"], p["beta"] = 0.75, -0.5
    ref, mag, _ = oracle_ref(p)
    for s in (1, 2, 4, 8, 16):
        say("case split", case[:3], "split_k", s)
        d1 = gemm_gpu(p, split_k=s)
        assert_parity(d1, ref, mag, "split %d" % s)
        d2 = gemm_gpu(p, split_k=s)
        assert np.array_equal(d1, d2), "split %d not reproducible" % s


@pytest.mark.parametrize("shape", [(1, 8192, 2048), (48, 1000, 1024), (512, 1024, 2048),
                                   (333, 777, 1312)])
def test_packed_b_matches_plain_b(shape, monkeypatch):
    M, N, K = shape
    p = inputs.make_problem(M, N, K, seed=0xBACC + N, beta=1.0, c_sigma=1.0)
    say("case packed", shape)
    ref, mag, _ = oracle_ref(p)
    if M == 1:
        # a row-major B at M == 1 runs the single-row GEMV, whose K order
        # differs from the skinny kernel's: against the oracle, then the
        # skinny kernel on both layouts
        assert_parity(gemm_gpu(p, split_k=1), ref, mag, "gemv")
        monkeypatch.setenv("MXGEMM_GEMV", "0")
    d_plain = gemm_gpu(p, split_k=1)
    d_packed = gemm_gpu(p, split_k=1, b_packed=True)
    assert np.array_equal(d_plain, d_packed)
    d_full = gemm_gpu(p, split_k=1, b_packed=True, sa_packed=True)
    assert np.array_equal(d_plain, d_full)
    assert_parity(d_packed, ref, mag, "packed")


def test_split_counters_survive_plan_changes():
    """Split-K calls with different tile counts on one stream, back to back:
    a call's partial sums must never be taken for another call's arrival
    counters (regression: they once shared one buffer)."""
    seq = [(63, 100, 4128, 8), (64, 4096, 2048, 2), (1, 64, 8192, 16), (700, 900, 2048, 4),
           (64, 4096, 2048, 2), (300, 520, 4096, 16), (1, 8192, 4096, 4)]
    for M, N, K, s in seq:
        p = inputs.make_problem(M, N, K, seed=0xC0C0 + M + N, beta=1.0, c_sigma=1.0)
        say("case counters", (M, N, K), "split", s)
        d = gemm_gpu(p, split_k=s)
        ref, mag, _ = oracle_ref(p)
        assert_parity(d, ref, mag, "sequence %s" % ((M, N, K, s),))


# (B and its scales packed, A scales packed)
PACK_MODES = [(False, False), (True, False), (True, True)]

EDGE_SHAPES = [
    (1, 1, 32), (1, 17, 96), (2, 5, 64), (15, 31, 160), (16, 16, 128), (17, 33, 288),
    (63, 100, 4128), (64, 4096, 2048), (65, 257, 544), (127, 129, 1056), (129, 130, 288),
    (300, 2048, 1024), (256, 256, 256), (257, 511, 2080), (1000, 40, 3232),
]


@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_edge_shapes(shape):
    M, N, K = shape
    p = inputs.make_problem(M, N, K, seed=0xED6E + M * 7 + N, e=(118, 136), beta=1.0, c_sigma=1.0)
    p["alpha"], p["beta"] = -1.25, 0.5
    ref, mag, _ = oracle_ref(p)
    for packed, sa_packed in PACK_MODES:
        say("case edge", shape, "packed", packed, sa_packed)
        d = gemm_gpu(p, b_packed=packed, sa_packed=sa_packed)
        assert_parity(d, ref, mag, "edge %s packed=%s,%s" % (shape, packed, sa_packed))


def test_identity_gives_A():
    """B = I (code 1.0 on the diagonal), unit scales: D == bf16(dequant A) exactly."""
    M, K = 128, 512
    p = inputs.make_problem(M, K, K, seed=0x1D, e=(120, 134))
    B = np.zeros((K, K // 2), dtype=np.uint8)
    for j in range(K):
        B[j, j // 2] |= (0x2 << 4) if (j & 1) else 0x2
    p["B"], p["SB"] = B, np.full((K, K // 32), 127, dtype=np.uint8)
    _, _, dref = oracle_ref(p)
    for packed in (False, True):
        d = gemm_gpu(p, b_packed=packed)
        same = (d == dref) | (((d | dref) & 0x7FFF) == 0)
        assert same.all()


def test_page_accuracy_profile():
    """With exponents 124..130 every product is exact in fp32; without split K
    the only error left is the bf16 output rounding, whose largest relative
    size is 2^-8/(1+2^-8) = 0.003891 -- the max_rel_err the asm_f4gemm README
    reports for all its kernels ("Verification")."""
    for M, N, K in [(256, 512, 1024), (1, 4096, 2048)]:
        p = inputs.make_problem(M, N, K, seed=0xACC + M, e=(124, 130))
        d = gemm_gpu(p, split_k=1)
        ref, mag, _ = oracle_ref(p)
        n_bad, _, rel = compare(d, ref, mag)
        assert n_bad == 0
        assert rel <= 2.0 ** -8 / (1 + 2.0 ** -8) + 1e-6, rel


def test_beta_zero_never_reads_C():
    M, N, K = 96, 200, 512
    p = inputs.make_problem(M, N, K, seed=0xC0, beta=1.0, c_sigma=1.0)
    p["beta"] = 0.0
    A, B, SA, SB = dev_u8(p["A"]), dev_u8(p["B"]), dev_u8(p["SA"]), dev_u8(p["SB"])
    C = dev_bf16(np.full((M, N), 0x7FC0, dtype=np.uint16))  # NaN
    ref, mag, _ = oracle_ref(p)
    for M_ in (M, 40):
        D = torch.empty((M_, N), dtype=torch.bfloat16, device="cuda")
        mx.mxgemm_run(D, C, A, B, SA, SB, 1.0, 0.0, M_, N, K)
        torch.cuda.synchronize()
        assert_parity(host_bits(D), ref[:M_], mag[:M_], "beta0")


def test_in_place_D_aliases_C():
    for M, N, K in [(200, 300, 1024), (8, 1000, 2048)]:
        p = inputs.make_problem(M, N, K, seed=0xA11A5 + M, beta=1.0, c_sigma=2.0)
        p["alpha"], p["beta"] = 2.0, -1.0
        ref, mag, _ = oracle_ref(p)
        A, B, SA, SB = dev_u8(p["A"]), dev_u8(p["B"]), dev_u8(p["SA"]), dev_u8(p["SB"])
        CD = dev_bf16(p["C"])
        mx.mxgemm_run(CD, CD, A, B, SA, SB, 2.0, -1.0, M, N, K)
        torch.cuda.synchronize()
        assert_parity(host_bits(CD), ref, mag, "in place")


@pytest.mark.parametrize("M", [40, 200])
def test_strided_operands(M):
    """Padded rows everywhere, odd scale pitch (byte-wise scale loads), scales
    at an odd address, D/C pitches that forbid vector stores."""
    N, K = 301, 1056
    p = inputs.make_problem(M, N, K, seed=0x57 + M, beta=1.0, c_sigma=1.0)
    p["alpha"], p["beta"] = 1.0, 1.0
    ref, mag, _ = oracle_ref(p)
    lda, ldb, ldsa, ldsb, ldc, ldd = K + 64, K + 96, K // 32 + 3, K // 32 + 5, N + 3, N + 1
    def pad(X, cols, fill):
        out = np.full((X.shape[0], cols), fill, dtype=X.dtype)
        out[:, : X.shape[1]] = X
        return out
    A = dev_u8(pad(p["A"], lda // 2, 0x77))
    B = dev_u8(pad(p["B"], ldb // 2, 0x77))
    SA_buf = dev_u8(np.concatenate([[0xFF], pad(p["SA"], ldsa, 0xFF).ravel()]))
    SB_buf = dev_u8(np.concatenate([[0xFF], pad(p["SB"], ldsb, 0xFF).ravel()]))
    C = dev_bf16(pad(p["C"], ldc, 0x7FC0))
    D = torch.zeros((M, ldd), dtype=torch.bfloat16, device="cuda")
    st = mx.make_strides(ldd=ldd, ldc=ldc, lda=lda, ldb=ldb, ldsa=ldsa, ldsb=ldsb)
    for s in (1, 4):
        mx.mxgemm_run(D, C, A, B, SA_buf.data_ptr() + 1, SB_buf.data_ptr() + 1, 1.0, 1.0, M, N, K,
                      strides=st, split_k=s)
        torch.cuda.synchronize()
        d = host_bits(D)
        assert_parity(d[:, :N], ref, mag, "strided split %d" % s)
        assert (d[:, N:] == 0).all()  # padding columns untouched


DEEP_SHAPES = [(65, 129, 128), (257, 511, 2048), (700, 300, 1152), (1000, 40, 384), (129, 1000, 640),
               (512, 512, 4096)]


@pytest.mark.parametrize("shape", DEEP_SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_tile_pipelines_agree(shape, monkeypatch):
    """Shapes with K % 128 == 0 and aligned scale rows can take the four-slot
    ring kernel; the two-stage kernel must give bit-identical results (same
    instruction sequence per accumulator), and both must match the oracle.
    Every tile shape is forced once per case, so each ring and two-stage
    instantiation runs."""
    M, N, K = shape
    p = inputs.make_problem(M, N, K, seed=0xDEE9 + M + N, e=(118, 136), beta=1.0, c_sigma=1.0)
    p["alpha"], p["beta"] = 0.5, 2.0
    ref, mag, _ = oracle_ref(p)
    for tile in range(4):
        monkeypatch.setenv("MXGEMM_FORCE_TILE", str(tile))
        for packed, sa_packed in PACK_MODES:
            for s in ((1, 2, 4) if tile == 0 else (1, 4)):
                say("case pipelines", shape, "tile", tile, "packed", packed, sa_packed, "split", s)
                monkeypatch.setenv("MXGEMM_TILE_PIPELINE", "deep")
                d_deep = gemm_gpu(p, split_k=s, b_packed=packed, sa_packed=sa_packed)
                monkeypatch.setenv("MXGEMM_TILE_PIPELINE", "two-stage")
                d_two = gemm_gpu(p, split_k=s, b_packed=packed, sa_packed=sa_packed)
                monkeypatch.delenv("MXGEMM_TILE_PIPELINE", raising=False)
                assert_parity(d_deep, ref, mag, "deep %s tile %d packed=%s,%s split=%d"
                              % (shape, tile, packed, sa_packed, s))
                assert np.array_equal(d_deep, d_two)


ROWS_CASES = [(17, 200, 2048), (40, 1000, 1056), (64, 333, 4096), (50, 4096, 8192), (33, 64, 512)]


@pytest.mark.parametrize("shape", ROWS_CASES, ids=lambda s: "%dx%dx%d" % s)
def test_rows_kernel_variants(shape):
    """16 < M <= 64 (the rows kernel): every operand packing, unsplit and
    split K, with ragged M, N and chunks that end inside a batch.  K = 1056
    leaves a K-block count that is not a multiple of 16, so the A scales take
    the per-wave load path; the other cases stage them through LDS."""
    M, N, K = shape
    p = inputs.make_problem(M, N, K, seed=0x2055 + M + N, dist="half_zero", e=(112, 140),
                            beta=1.0, c_sigma=1.0)
    p["alpha"], p["beta"] = 1.5, -0.75
    ref, mag, _ = oracle_ref(p)
    assert mx.mxgemm_plan(M, N, K, 0, 1, 256)["kernel_name"].startswith("rows_m%dx16" % -(-M // 16))
    for packed, sa_packed in PACK_MODES:
        outs = []
        for s in (1, 2, 4):
            say("case rows", shape, "packed", packed, sa_packed, "split", s)
            d = gemm_gpu(p, split_k=s, b_packed=packed, sa_packed=sa_packed)
            assert_parity(d, ref, mag, "rows %s packed=%s,%s split=%d" % (shape, packed, sa_packed, s))
            outs.append(d)
        assert np.array_equal(gemm_gpu(p, split_k=4, b_packed=packed, sa_packed=sa_packed), outs[2])


LEAN_CASES = [(17, 16500, 1024, 1), (40, 20000, 1056, 1), (64, 17000, 2048, 1), (50, 8200, 2048, 4)]


@pytest.mark.parametrize("case", LEAN_CASES, ids=lambda c: "%dx%dx%d_split%d" % c)
def test_rows_lean_ring(case):
    """More workgroups than CUs with row-major B: the rows kernel with a
    two-slot ring (two workgroups per CU) for every 16-row group count,
    A scales staged (K-block count a multiple of 16) and per wave (K =
    1056), unsplit and split K; the same values as the packed-B launch,
    which keeps the four-slot ring."""
    M, N, K, s = case
    p = inputs.make_problem(M, N, K, seed=0x1EA4 + M + N, dist="half_zero", e=(112, 140),
                            beta=1.0, c_sigma=1.0)
    p["alpha"], p["beta"] = 1.5, -0.75
    ref, mag, _ = oracle_ref(p)
    name = mx.mxgemm_plan(M, N, K, 0, s, 256)["kernel_name"]
    assert name == "rows_m%dx16_n4x1x16_u4_r2" % -(-M // 16), name
    assert mx.mxgemm_plan(M, N, K, 1, s, 256)["kernel_name"].endswith("_r4")
    say("case rows lean", case)
    d = gemm_gpu(p, split_k=s)
    assert_parity(d, ref, mag, "rows lean %s" % (case,))
    assert np.array_equal(gemm_gpu(p, split_k=s, b_packed=True), d)

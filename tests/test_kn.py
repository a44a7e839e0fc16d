"""GPU parity of MN-major B (b_layout = MXGEMM_B_KN), through the C-ABI.

B's codes are stored [K][ldb/2]: row k holds the N columns' codes at that k
("CDNA4 MFMA transpose load builtins", opening section: a B tile kept
row-major).  The tiled kernel stages such tiles into LDS unchanged and forms
each 16 x 128 operand from two ds_read_tr4_b64 (K-rows 32g..32g+15 and
32g+16..32g+31 of lane group g, the K split of that page's "Hardware
constraints" table).  Every case is compared element by element with the
oracle reading the same MN-major bytes, and -- where the K-major call runs
the same tile and split on the tiled kernel -- bit for bit with the K-major
result (same matrix instructions in the same order).  Cases: ragged M, N
and K (K-block counts that are not multiples of 8), M = 1, every tile
shape, row-major and packed B scales, packed A scales, split 1/2/4, row
pitches wider than N holding large codes that must never be read, and the
8192^3 shape, and the persistent form against its plain grid.
"""
import os
import sys

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
import oracle
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxgpu import assert_parity, dev_bf16, dev_u8, gemm_gpu, host_bits, oracle_ref  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def lib_loaded():
    mx.lib()
    yield
    mx.mxgemm_release_workspaces()


def kn_problem(M, N, K, seed, extra=0, **kw):
    p = inputs.make_problem(M, N, K, seed=seed, **kw)
    ldb = -(-N // 32) * 32 + extra
    p["B_kn"] = inputs.to_mn_major(p["B"], N, K, ldb, pad=0x7)  # padding columns hold 6.0
    p["ldb_kn"] = ldb
    return p


def k_major(p):
    q = dict(p)
    q["B_kn"] = None
    return q


MODES = [(False, False), (True, False), (True, True)]  # (B scales packed, A scales packed)
SHAPES = [(1, 256, 512), (5, 40, 1056), (17, 200, 2048), (64, 7168, 2048), (129, 130, 288), (300, 520, 4096),
          (257, 511, 2080), (1000, 40, 3232), (512, 1024, 2048)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_mn_major_parity(shape):
    M, N, K = shape
    p = kn_problem(M, N, K, seed=0x4B + M + N, e=(116, 138), beta=1.0, c_sigma=1.0, extra=32 * (M % 3))
    p["alpha"], p["beta"] = -1.25, 0.5
    ref, mag, _ = oracle_ref(p)
    for sbp, sap in MODES:
        for s in (1, 4):
            say("case kn", shape, "sb packed", sbp, "sa packed", sap, "split", s)
            d = gemm_gpu(p, split_k=s, b_packed=sbp, sa_packed=sap)
            assert_parity(d, ref, mag, "kn %s sb=%s sa=%s split=%d" % (shape, sbp, sap, s))
            if M > 64 and s == 1:
                assert np.array_equal(d, gemm_gpu(k_major(p), split_k=s, b_packed=sbp, sa_packed=sap))


@pytest.mark.parametrize("tile", [0, 1, 2, 3])
def test_mn_major_every_tile_matches_k_major(tile, monkeypatch):
    monkeypatch.setenv("MXGEMM_FORCE_TILE", str(tile))
    monkeypatch.setenv("MXGEMM_TILE_PIPELINE", "two-stage")
    for M, N, K in [(300, 520, 2048), (257, 511, 2080), (96, 96, 1024)]:
        p = kn_problem(M, N, K, seed=0x7E1 + tile + N, e=(118, 136))
        ref, mag, _ = oracle_ref(p)
        for sbp, sap in MODES:
            for s in (1, 2):
                say("case kn tile", tile, (M, N, K), "sb packed", sbp, "sa packed", sap, "split", s)
                d = gemm_gpu(p, split_k=s, b_packed=sbp, sa_packed=sap)
                assert_parity(d, ref, mag, "kn tile %d %s" % (tile, (M, N, K, sbp, sap, s)))
                assert np.array_equal(d, gemm_gpu(k_major(p), split_k=s, b_packed=sbp, sa_packed=sap))


def test_mn_major_square_8192(monkeypatch):
    """The headline shape with an MN-major B (packed scales): bit-identical
    to the K-major fully packed result, and sampled rows against the oracle."""
    M = N = K = 8192
    p = kn_problem(M, N, K, seed=0x8192)
    say("case kn 8192^3")
    d = gemm_gpu(p, split_k=-1, b_packed=True, sa_packed=True)
    d0 = gemm_gpu(k_major(p), split_k=-1, b_packed=True, sa_packed=True)
    assert np.array_equal(d, d0), "%d elements differ from the K-major result" % int((d != d0).sum())
    rows = np.array([0, 1, 255, 256, 4095, 8191], dtype=np.int64)
    ref, mag, _ = oracle_ref(p, rows=rows)
    assert_parity(d[rows], ref, mag, "kn 8192^3")


def test_mn_major_persistent_matches_plain_grid(monkeypatch):
    """MN-major B with packed scales on 400 whole 256 x 256 tiles (an uneven
    last round on 256 CUs): the persistent form equals the plain grid and the
    K-major result bit for bit, and sampled rows match the oracle."""
    M = N = 5120
    K = 512
    p = kn_problem(M, N, K, seed=0x5120)
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=p["ldb_kn"], ldsa=K // 32, ldsb=K // 32, b_packed=1, sa_packed=1,
                         b_layout=mx.B_KN)
    assert mx.mxgemm_query_ex(M, N, K, st, -1)["persist_grid"] > 0
    say("case kn persistent")
    d = gemm_gpu(p, split_k=-1, b_packed=True, sa_packed=True)
    monkeypatch.setenv("MXGEMM_TILE_PERSIST", "0")
    say("case kn plain grid")
    d_plain = gemm_gpu(p, split_k=-1, b_packed=True, sa_packed=True)
    monkeypatch.delenv("MXGEMM_TILE_PERSIST")
    assert np.array_equal(d, d_plain), "%d elements differ from the plain grid" % int((d != d_plain).sum())
    assert np.array_equal(d, gemm_gpu(k_major(p), split_k=-1, b_packed=True, sa_packed=True))
    rows = np.array([0, 255, 256, 2600, M - 1], dtype=np.int64)
    ref, mag, _ = oracle_ref(p, rows=rows)
    assert_parity(d[rows], ref, mag, "kn persistent")


def test_mn_major_strides_and_offsets():
    """Row pitches wider than N (padding holds code 0x7 = 6.0 and must never
    be read), scales at odd addresses with odd pitches, D and C pitches that
    forbid vector stores."""
    M, N, K = 200, 301, 1056
    p = kn_problem(M, N, K, seed=0x57D, beta=1.0, c_sigma=1.0, extra=96)
    p["alpha"], p["beta"] = 1.0, 1.0
    ref, mag, _ = oracle_ref(p)
    ldsa, ldsb, ldc, ldd = K // 32 + 3, K // 32 + 5, N + 3, N + 1

    def pad(X, cols, fill):
        out = np.full((X.shape[0], cols), fill, dtype=X.dtype)
        out[:, : X.shape[1]] = X
        return out
    A = dev_u8(p["A"])
    B = dev_u8(p["B_kn"])
    SA_buf = dev_u8(np.concatenate([[0xFF], pad(p["SA"], ldsa, 0xFF).ravel()]))
    SB_buf = dev_u8(np.concatenate([[0xFF], pad(p["SB"], ldsb, 0xFF).ravel()]))
    C = dev_bf16(pad(p["C"], ldc, 0x7FC0))
    D = torch.zeros((M, ldd), dtype=torch.bfloat16, device="cuda")
    st = mx.make_strides(ldd=ldd, ldc=ldc, lda=K, ldb=p["ldb_kn"], ldsa=ldsa, ldsb=ldsb, b_layout=mx.B_KN)
    for s in (1, 4):
        mx.mxgemm_run(D, C, A, B, SA_buf.data_ptr() + 1, SB_buf.data_ptr() + 1, 1.0, 1.0, M, N, K,
                      strides=st, split_k=s)
        torch.cuda.synchronize()
        d = host_bits(D)
        assert_parity(d[:, :N], ref, mag, "kn strided split %d" % s)
        assert (d[:, N:] == 0).all()


@pytest.mark.parametrize("M", [1, 40])
def test_mn_major_from_bf16_activations(M):
    """mxgemm_run_bf16a with an MN-major B quantizes first (also at M = 1):
    bit for bit mxgemm_quantize followed by mxgemm_run."""
    N, K = 520, 2048
    rng = np.random.default_rng(M)
    xbits = inputs.f32_to_bf16_bits((rng.standard_normal((M, K)) * 4).astype(np.float32))
    X = dev_bf16(xbits)
    p = kn_problem(M, N, K, seed=0xB16 + M)
    B, SB = dev_u8(p["B_kn"]), dev_u8(p["SB"])
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=p["ldb_kn"], ldsa=K // 32, ldsb=K // 32, b_layout=mx.B_KN)
    D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mx.mxgemm_run_bf16a(D, None, X, B, SB, 1.0, 0.0, M, N, K, strides=st)
    A = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    SA = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    mx.mxgemm_quantize(A, SA, X, M, K)
    D2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mx.mxgemm_run(D2, None, A, B, SA, SB, 1.0, 0.0, M, N, K, strides=st)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(D), host_bits(D2))
    p["A"], p["SA"] = oracle.quantize_mxfp4(xbits)  # the oracle's own quantization
    ref, mag, _ = oracle_ref(p)
    assert_parity(host_bits(D), ref, mag, "kn bf16a M=%d" % M)

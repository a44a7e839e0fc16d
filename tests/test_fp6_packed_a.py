"""GPU parity of a pre-packed FP6 A (mxgemm_pack_a, then mxgemm_run with
a_packed = 1), through the C-ABI.

mxgemm_pack_a performs, once, the re-layout mxgemm_run applies to a
row-major FP6 A on every call with M > 64 (the scaled instruction's operand
order, "CDNA4 dense MFMA builtins", "Mixed-precision with scaling"; the A
scales in the asm_f4gemm README's "A_scale / B_scale" shuffle).  The dense
FP6 tile then reads the caller's copy: D must equal the row-major call on
the same tile bit for bit (same operands, same instructions in the same
order) and the oracle element by element.  Cases: both FP6 formats, ragged M
and N, a K tail of 33 blocks, split 1 and 2, packed and row-major B, C with
beta, the persistent grid (5120 x 5120), the allocation-free entry point.
"""
import sys

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxgpu import assert_parity, dev_bf16, dev_u8, host_bits, oracle_ref  # noqa: E402

NAMES = {3: "e2m3", 4: "e3m2"}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def lib_loaded():
    mx.lib()
    yield
    mx.mxgemm_release_workspaces()


def problem(M, N, K, fmt, seed, beta):
    p = inputs.make_problem(M, N, K, seed=seed, e=(120, 134), beta=beta, c_sigma=2.0 if beta else None,
                            a_fmt=fmt)
    p["alpha"] = 0.5
    if beta:
        p["beta"] = -0.75
    return p


def run(p, split, packed_b, a_packed, entry=None):
    """D for problem p: A row-major (a_packed False) or through mxgemm_pack_a."""
    M, N, K, fmt = p["M"], p["N"], p["K"], p["a_fmt"]
    A, SA, B, SB = dev_u8(p["A"]), dev_u8(p["SA"]), dev_u8(p["B"]), dev_u8(p["SB"])
    if packed_b:
        info = mx.mxgemm_plan(M, N, K, 1, -1, 256)
        Bp = torch.empty(info["packed_b_bytes"], dtype=torch.uint8, device="cuda")
        SBp = torch.empty(info["packed_sb_bytes"], dtype=torch.uint8, device="cuda")
        mx.mxgemm_pack_b(Bp, SBp, B, SB, N, K)
        B, SB = Bp, SBp
    if a_packed:
        Ap = torch.full((mx.mxgemm_pack_a_bytes(M, K),), 0xA5, dtype=torch.uint8, device="cuda")
        SAp = torch.full((mx.mxgemm_plan(M, N, K, 1, -1, 256)["packed_sa_bytes"],), 0xFF, dtype=torch.uint8,
                         device="cuda")
        mx.mxgemm_pack_a(Ap, SAp, A, SA, M, K, fmt)
        A, SA = Ap, SAp
    C = dev_bf16(p["C"]) if p["beta"] != 0.0 else None
    D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, b_packed=int(packed_b),
                         a_format=fmt, a_packed=int(a_packed))
    (entry or mx.mxgemm_run)(D, C, A, B, SA, SB, p["alpha"], p["beta"], M, N, K, strides=st, split_k=split)
    torch.cuda.synchronize()
    return host_bits(D)


# (M, N, K, split, packed B, beta)
CASES = [
    (300, 520, 1056, 1, False, 1.0),
    (1000, 777, 2048, 2, True, 0.0),
    (4096, 4096, 1024, 1, True, 0.0),
]


@pytest.mark.parametrize("fmt", [3, 4], ids=lambda f: NAMES[f])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%dx%d_s%d%s%s" % (
    c[0], c[1], c[2], c[3], "_packed" if c[4] else "", "_c" if c[5] else ""))
def test_prepacked_A_matches_rowmajor_call(case, fmt, monkeypatch):
    M, N, K, split, packed_b, beta = case
    p = problem(M, N, K, fmt, seed=0xA6A6 + 7 * fmt + M + N, beta=beta)
    # the row-major call on the same (dense FP6) tile
    monkeypatch.setenv("MXGEMM_A8_TILE", "tile_fp6_256x256")
    say("case prepacked fp6 A", NAMES[fmt], case)
    d_rows = run(p, split, packed_b, False)
    d = run(p, split, packed_b, True)
    assert np.array_equal(d, d_rows), "%d of %d elements differ" % (int((d != d_rows).sum()), d.size)
    rows = None if M * N * K <= (1 << 31) else np.sort(np.random.default_rng(M).choice(M, 64, replace=False))
    ref, mag, _ = oracle_ref(p, rows=rows)
    assert_parity(d if rows is None else d[rows], ref, mag, "prepacked fp6 %s %s" % (NAMES[fmt], case))


def test_prepacked_A_persistent_and_noalloc():
    """5120 x 5120 x 512 (400 tiles, the persistent grid) with packed B: the
    pre-packed call equals the row-major call, and the allocation-free entry
    point equals mxgemm_run on it."""
    M = N = 5120
    K = 512
    fmt = 3
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, b_packed=1, a_format=fmt,
                         a_packed=1)
    info = mx.mxgemm_query_ex(M, N, K, st, -1)
    assert info["kernel_name"] == "tile_fp6_256x256" and info["persist_grid"] > 0, info
    p = problem(M, N, K, fmt, seed=0xA6F0, beta=0.0)
    say("case prepacked fp6 A persistent")
    d = run(p, -1, True, True)
    assert np.array_equal(d, run(p, -1, True, False))
    assert np.array_equal(d, run(p, -1, True, True, entry=mx.mxgemm_run_noalloc))
    rows = np.array([0, 1, 255, 256, 2047, 4095, 5119])
    ref, mag, _ = oracle_ref(p, rows=rows)
    assert_parity(d[rows], ref, mag, "prepacked fp6 persistent")

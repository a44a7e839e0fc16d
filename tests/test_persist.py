"""GPU parity of the persistent form of the tiled kernel, through the C-ABI.

The persistent form (one workgroup per CU walking its tiles, the next tile's
first stage loaded while the last tile's D is written) runs the same matrix
instructions in the same order as the plain grid, so D must match the plain
grid's bit for bit (MXGEMM_TILE_PERSIST=0 selects it), and sampled rows and
columns must match the oracle.  The persistent tiles are FP4 256 x 256 with
packed B and A scales, and the dense FP6 256 x 256 tile (B packed by the
caller or by the library); cases cover an uneven last round (400 tiles on
256 CUs), two and four whole rounds, and the 8192^3 shape.
"""
import os
import sys

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxgpu import assert_parity, gemm_gpu, oracle_ref  # noqa: E402

# (M, N, K, a_format, tile, layouts that run persistent)
CASES = [
    (5120, 5120, 512, 0, (256, 256), [(True, True)]),
    (4096, 8192, 1024, 0, (256, 256), [(True, True)]),
    (8192, 8192, 1024, 0, (256, 256), [(True, True)]),
    (8192, 8192, 8192, 0, (256, 256), [(True, True)]),
    (5120, 5120, 512, 3, (256, 256), [(True, False), (False, False)]),
    (4096, 8192, 1024, 4, (256, 256), [(True, False), (False, False)]),
]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def plan(M, N, K, fmt, packed, sa_packed):
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32,
                         b_packed=int(packed), sa_packed=int(sa_packed), a_format=fmt)
    return mx.mxgemm_query_ex(M, N, K, st, -1)


def plain_grid(p, **kw):
    old = os.environ.get("MXGEMM_TILE_PERSIST")
    os.environ["MXGEMM_TILE_PERSIST"] = "0"
    try:
        return gemm_gpu(p, **kw)
    finally:
        if old is None:
            del os.environ["MXGEMM_TILE_PERSIST"]
        else:
            os.environ["MXGEMM_TILE_PERSIST"] = old


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%dx%d_f%d" % c[:4])
def test_persistent_matches_plain_grid_and_oracle(case):
    M, N, K, fmt, tile, layouts = case
    e = (110, 130) if fmt in (1, 2) else (118, 136)
    p = inputs.make_problem(M, N, K, seed=0x9E51 + M + N + K + fmt, e=e, a_fmt=fmt)
    p["alpha"] = -0.75
    rng = np.random.default_rng(M + N + fmt)
    rows = np.sort(np.concatenate([[0, 127, 128, 255, 256, M - 256, M - 1], rng.choice(M, 9, replace=False)]))
    cols = np.sort(np.concatenate([[0, 127, 128, 255, 256, N - 256, N - 1], rng.choice(N, 25, replace=False)]))
    ref, mag, _ = oracle_ref(p, rows=rows, cols=cols)
    for packed, sa_packed in layouts:
        info = plan(M, N, K, fmt, packed, sa_packed)
        assert (info["tile_m"], info["tile_n"]) == tile and info["persist_grid"] > 0, info
        say("case persistent", case[:4], "packed", packed, sa_packed, info["kernel_name"])
        d = gemm_gpu(p, split_k=-1, b_packed=packed, sa_packed=sa_packed)
        say("case plain grid", case[:4], "packed", packed, sa_packed)
        d0 = plain_grid(p, split_k=-1, b_packed=packed, sa_packed=sa_packed)
        assert np.array_equal(d, d0), "%d elements differ from the plain grid" % int((d != d0).sum())
        assert_parity(d[np.ix_(rows, cols)], ref, mag, "persistent %s %s,%s" % (case[:4], packed, sa_packed))


def test_persistent_runs_back_to_back_with_other_shapes():
    """Persistent and plain launches interleaved on one stream: nothing a
    persistent launch leaves behind (LDS, counters) reaches the next call."""
    seq = [(5120, 5120, 512), (300, 520, 1024), (4096, 8192, 1024), (256, 256, 256), (5120, 5120, 512)]
    for M, N, K in seq:
        p = inputs.make_problem(M, N, K, seed=0xB2B + M + K)
        say("case sequence", (M, N, K))
        d = gemm_gpu(p, b_packed=True, sa_packed=True)
        rows = np.unique(np.linspace(0, M - 1, 9).astype(np.int64))
        cols = np.unique(np.linspace(0, N - 1, 33).astype(np.int64))
        ref, mag, _ = oracle_ref(p, rows=rows, cols=cols)
        assert_parity(d[np.ix_(rows, cols)], ref, mag, "sequence %s" % ((M, N, K),))

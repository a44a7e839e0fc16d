"""GPU parity of the persistent form of the 256 x 256 tiled kernel, through
the C-ABI.

The persistent form (one workgroup per CU walking its tiles, the next tile's
first stage loaded while the last tile's D is written) runs the same matrix
instructions in the same order as the plain grid, so D must match the plain
grid's bit for bit (MXGEMM_TILE_PERSIST=0 selects it), and sampled rows and
columns must match the oracle.  Shapes cover an uneven last round (400 tiles
on 256 CUs), two full rounds, four rounds (the 8192 x 8192 output) and every
operand packing.
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

PACK_MODES = [(False, False), (True, False), (True, True)]
SHAPES = [(5120, 5120, 512), (4096, 8192, 1024), (8192, 8192, 1024)]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def persist_grid(M, N, K, packed, sa_packed):
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32,
                         b_packed=int(packed), sa_packed=int(sa_packed))
    return mx.mxgemm_query_ex(M, N, K, st, -1)["persist_grid"]


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


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_persistent_matches_plain_grid_and_oracle(shape):
    M, N, K = shape
    p = inputs.make_problem(M, N, K, seed=0x9E51 + M + N + K, e=(118, 136))
    p["alpha"] = -0.75
    rng = np.random.default_rng(M + N)
    rows = np.sort(np.concatenate([[0, 255, 256, M - 256, M - 1], rng.choice(M, 11, replace=False)]))
    cols = np.sort(np.concatenate([[0, 255, 256, N - 256, N - 1], rng.choice(N, 27, replace=False)]))
    ref, mag, _ = oracle_ref(p, rows=rows, cols=cols)
    for packed, sa_packed in PACK_MODES:
        assert persist_grid(M, N, K, packed, sa_packed) > 0
        say("case persistent", shape, "packed", packed, sa_packed)
        d = gemm_gpu(p, split_k=-1, b_packed=packed, sa_packed=sa_packed)
        say("case plain grid", shape, "packed", packed, sa_packed)
        d0 = plain_grid(p, split_k=-1, b_packed=packed, sa_packed=sa_packed)
        assert np.array_equal(d, d0), "%d elements differ from the plain grid" % int((d != d0).sum())
        assert_parity(d[np.ix_(rows, cols)], ref, mag, "persistent %s %s,%s" % (shape, packed, sa_packed))


def test_persistent_runs_back_to_back_with_other_shapes():
    """Persistent and plain launches interleaved on one stream: nothing a
    persistent launch leaves behind (LDS, counters) reaches the next call."""
    seq = [(5120, 5120, 512), (300, 520, 1024), (4096, 8192, 1024), (256, 256, 256), (5120, 5120, 512)]
    for M, N, K in seq:
        p = inputs.make_problem(M, N, K, seed=0xB2B + M + K)
        say("case sequence", (M, N, K))
        d = gemm_gpu(p)
        rows = np.unique(np.linspace(0, M - 1, 9).astype(np.int64))
        cols = np.unique(np.linspace(0, N - 1, 33).astype(np.int64))
        ref, mag, _ = oracle_ref(p, rows=rows, cols=cols)
        assert_parity(d[np.ix_(rows, cols)], ref, mag, "sequence %s" % ((M, N, K),))

"""GPU parity of the headline workload on every output element.

The 8192 x 8192 x 8192 square workload runs as the benchmark times it (B
and both scale matrices pre-shuffled, the persistent 256 x 256 tiled
kernel, split 1, beta = 0) and all 67,108,864 elements of D are compared
with the oracle (threaded over output columns; about 5.5e11 fp64 products,
tens of seconds on the host's cores), row block by row block, under the
tolerance of tests/mxgpu.py.
"""
import sys
import time

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxgpu import assert_parity, gemm_gpu, oracle_ref  # noqa: E402


@pytest.mark.timeout(1800)
def test_square_8192_every_element():
    mx.lib()
    p = inputs.make_workload("square_8192")
    M, N, K = p["M"], p["N"], p["K"]
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, b_packed=1, sa_packed=1)
    info = mx.mxgemm_query_ex(M, N, K, st, -1)
    assert info["persist_grid"] > 0 and info["split_k"] == 1, info
    print("case full square_8192", info["kernel_name"], file=sys.stderr, flush=True)
    d = gemm_gpu(p, split_k=-1, b_packed=True, sa_packed=True)
    mx.mxgemm_release_workspaces()
    t0 = time.perf_counter()
    worst = 0.0
    for r0 in range(0, M, 512):
        rows = np.arange(r0, min(M, r0 + 512), dtype=np.int64)
        ref, mag, _ = oracle_ref(p, rows=rows)
        worst = max(worst, assert_parity(d[rows], ref, mag, "square_8192 rows %d.." % r0))
        print("  rows %d..%d ok (%.0f s)" % (r0, rows[-1], time.perf_counter() - t0), file=sys.stderr, flush=True)
    print("  max rel err %.4g over %d elements" % (worst, M * N), file=sys.stderr, flush=True)

"""mxgemm_run_noalloc through the C-ABI: the allocation-free form of
mxgemm_run (split-K counters and partials, and FP6 A's re-laid copy, in the
library's fixed per-device scratch) gives mxgemm_run's output bit for bit,
on consecutive calls whose second is smaller (the scratch keeps the first
call's contents), refuses plans beyond the scratch before launching
anything, and replays correctly from a HIP graph."""
import sys

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxgpu import assert_parity, dev_bf16, dev_u8, host_bits, oracle_ref  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def operands(p):
    M, N, K = p["M"], p["N"], p["K"]
    C = dev_bf16(p["C"]) if p.get("C") is not None else None
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, a_format=int(p.get("a_fmt", 0)))
    return dict(A=dev_u8(p["A"]), B=dev_u8(p["B"]), SA=dev_u8(p["SA"]), SB=dev_u8(p["SB"]), C=C, st=st)


def run(fn, p, ops, split, D=None):
    M, N, K = p["M"], p["N"], p["K"]
    if D is None:
        D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    fn(D, ops["C"] if p["beta"] != 0.0 else None, ops["A"], ops["B"], ops["SA"], ops["SB"], p["alpha"], p["beta"],
       M, N, K, strides=ops["st"], split_k=split)
    torch.cuda.synchronize()
    return host_bits(D)


# (M, N, K, split, A format): the skinny split path, the rows kernel's split,
# the tiled split, FP6 A on the 8-bit tiles (its re-laid copy in the
# scratch), the rows kernel's split with FP8 and FP6 A, the rows kernel's
# two-slot ring (516 workgroups) split, the single-row GEMV (no scratch)
# with FP4 and FP8 A; each is followed by a smaller call
CASES = [
    [(64, 7168, 16384, 2, 0), (40, 1000, 2048, 4, 0)],
    [(300, 520, 4096, 4, 0), (17, 200, 2048, 2, 0)],
    [(1, 8192, 8192, 16, 0), (1, 300, 4096, 4, 0)],
    [(300, 520, 2048, 2, 3), (100, 260, 1024, 1, 3)],
    [(64, 2048, 4096, 2, 1), (33, 500, 2048, 4, 3)],
    [(50, 8200, 2048, 4, 0), (40, 1000, 1024, 2, 0)],
    [(1, 8192, 8192, -1, 0), (1, 2050, 4096, -1, 1)],
]


@pytest.mark.parametrize("seq", CASES, ids=lambda s: "%dx%dx%d" % s[0][:3])
def test_noalloc_matches_run_on_consecutive_calls(seq):
    mx.lib()
    for M, N, K, split, fmt in seq:
        p = inputs.make_problem(M, N, K, seed=0xA110C + M + N + fmt, e=(112, 140), beta=1.0, c_sigma=2.0,
                                a_fmt=fmt, dist="half_zero" if fmt == 0 else "uniform")
        p["alpha"], p["beta"] = 0.75, -0.5
        ops = operands(p)
        say("case noalloc", (M, N, K), "split", split, "a_format", fmt)
        d_ref = run(mx.mxgemm_run, p, ops, split)
        d = run(mx.mxgemm_run_noalloc, p, ops, split)
        assert np.array_equal(d, d_ref), "%d of %d elements differ from mxgemm_run" % (int((d != d_ref).sum()), d.size)
        cols = np.arange(N) if M * N * K <= 2 ** 31 else np.arange(0, N, 37)
        ref, mag, _ = oracle_ref(p, cols=cols)
        assert_parity(d[:, cols], ref, mag, "noalloc %s" % ((M, N, K, split, fmt),))


def test_noalloc_fp6_dense_tile(monkeypatch):
    """The dense FP6 tile (forced through the planner's test hook) keeps its
    re-laid A, shuffled A scales and the packed copy of a row-major B in the
    scratch: bit for bit mxgemm_run's output on two consecutive calls, the
    second smaller."""
    mx.lib()
    monkeypatch.setenv("MXGEMM_A8_TILE", "tile_fp6_256x256")
    for M, N, K, split, fmt in [(512, 520, 2048, 1, 3), (300, 300, 1056, 2, 4)]:
        p = inputs.make_problem(M, N, K, seed=0xD6A1 + M + fmt, e=(118, 136), beta=1.0, c_sigma=2.0, a_fmt=fmt)
        p["alpha"], p["beta"] = 0.75, -0.5
        ops = operands(p)
        assert mx.mxgemm_plan_ex(M, N, K, ops["st"], split, 256)["kernel_name"] == "tile_fp6_256x256"
        say("case noalloc fp6 dense", (M, N, K), "split", split, "a_format", fmt)
        d_ref = run(mx.mxgemm_run, p, ops, split)
        d = run(mx.mxgemm_run_noalloc, p, ops, split)
        assert np.array_equal(d, d_ref), "%d of %d elements differ from mxgemm_run" % (int((d != d_ref).sum()), d.size)
        ref, mag, _ = oracle_ref(p)
        assert_parity(d, ref, mag, "noalloc fp6 dense %s" % ((M, N, K, split, fmt),))


def test_noalloc_refuses_plans_beyond_its_scratch():
    mx.lib()
    M, N, K = 4096, 4096, 8192
    p = inputs.make_problem(M, N, K, seed=0xB16)
    ops = operands(p)
    info = mx.mxgemm_query_ex(M, N, K, ops["st"], 16)
    assert info["workspace_bytes"] > mx.NOALLOC_SCRATCH_BYTES, info
    D = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    st = mx.mxgemm_run_noalloc(D, None, ops["A"], ops["B"], ops["SA"], ops["SB"], 1.0, 0.0, M, N, K,
                               strides=ops["st"], split_k=16, check=False)
    torch.cuda.synchronize()
    assert st == -7
    assert int(torch.count_nonzero(D)) == 0  # nothing launched
    # with the caller's workspace only the counters come from the scratch
    ws = torch.empty(info["workspace_bytes"], dtype=torch.uint8, device="cuda")
    st2 = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, workspace=ws,
                          workspace_bytes=ws.numel())
    mx.mxgemm_run_noalloc(D, None, ops["A"], ops["B"], ops["SA"], ops["SB"], 1.0, 0.0, M, N, K,
                          strides=st2, split_k=16)
    torch.cuda.synchronize()
    rows = np.arange(0, M, 511)
    ref, mag, _ = oracle_ref(p, rows=rows)
    assert_parity(host_bits(D)[rows], ref, mag, "noalloc with caller workspace")


def test_noalloc_replays_from_a_graph():
    """Captured once, replayed five times with eager work and
    synchronizations in between; every replay equals the eager result."""
    mx.lib()
    M, N, K, split = 64, 4096, 8192, 4
    p = inputs.make_problem(M, N, K, seed=0x6A9, e=(118, 136), beta=1.0, c_sigma=1.0)
    ops = operands(p)
    d_eager = run(mx.mxgemm_run, p, ops, split)
    D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):  # first call on the device outside the capture
        mx.mxgemm_run_noalloc(D, ops["C"], ops["A"], ops["B"], ops["SA"], ops["SB"], p["alpha"], p["beta"],
                              M, N, K, strides=ops["st"], split_k=split, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mx.mxgemm_run_noalloc(D, ops["C"], ops["A"], ops["B"], ops["SA"], ops["SB"], p["alpha"], p["beta"],
                              M, N, K, strides=ops["st"], split_k=split, stream=s)
    for i in range(5):
        D.fill_(float("nan"))
        run(mx.mxgemm_run, p, ops, 2)  # other work on the default stream in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(D), d_eager), "replay %d" % i

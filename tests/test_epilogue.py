"""GPU parity of mxgemm_run's epilogue options, through the C-ABI.

- A float32 C (c_f32 = 1): the f32 bias operand that the asm_f4gemm
  README's "C / bias" note says aiter documents.  Every kernel family
  (tiled two-stage and four-slot ring, skinny M <= 16, rows 16 < M <= 64),
  split and unsplit, against the oracle's exact fp64 reference; and with
  A = 0, D must be bf16(beta * C) bit for bit, which only holds if C is read
  at full f32 precision.
- The opt-in bf16-atomic split-K (split_mode = 1), measured against the
  README's "Verification" table: split-K error of aiter's kernels on
  M = 256, N = 1024, K = 4096 with operand exponents 2^-3 .. 2^3, as max
  |D - ref| over max |ref|.  The README bounds it by 2 % of max |ref|; the
  default fp32 reduction must stay within the per-element tolerance at
  every split.
"""
import sys

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxgpu import assert_parity, bf16_to_f64, gemm_gpu, oracle_ref  # noqa: E402

# README "Verification" table: log2_k_split -> max abs err / max|ref| (%)
PAGE_SPLIT_ERR = {1: 0.28, 2: 0.51, 4: 0.62, 8: 0.81, 16: 1.15}
PAGE_BOUND = 0.02


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# (M, N, K, split, b_packed): which kernel the planner picks is checked below
F32_CASES = [
    (300, 520, 1024, 1, False),   # tiled
    (300, 520, 1024, 4, True),    # tiled, split, packed B
    (128, 256, 512, 1, False),    # small tile (four-slot ring)
    (1, 1000, 2048, 1, False),    # skinny, single-row A
    (8, 777, 4096, 4, False),     # skinny, split, ragged N
    (40, 1000, 1056, 2, False),   # rows kernel, split, K tail
    (64, 333, 4096, 1, True),     # rows kernel, packed B
]


def f32_problem(M, N, K, seed):
    p = inputs.make_problem(M, N, K, seed=seed, beta=1.0, c_sigma=1.0)
    rng = np.random.default_rng(seed ^ 0xF32)
    # f32 values with all 24 mantissa bits in use (no bf16 value among them)
    p["C"] = (rng.standard_normal((M, N)) * 4.0).astype(np.float32)
    p["beta"] = -0.5
    return p


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "%dx%dx%d_s%d%s" % (c[:4] + ("_packed" if c[4] else "",)))
def test_f32_C_matches_oracle(case):
    M, N, K, split, packed = case
    p = f32_problem(M, N, K, seed=0x5EED + M * 3 + N)
    say("case f32 C", case, mx.mxgemm_plan(M, N, K, int(packed), split, 256)["kernel_name"])
    d = gemm_gpu(p, split_k=split, b_packed=packed)
    ref, mag, _ = oracle_ref(p)
    assert_parity(d, ref, mag, "f32 C %s" % (case,))


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "%dx%dx%d_s%d%s" % (c[:4] + ("_packed" if c[4] else "",)))
def test_f32_C_is_read_at_full_precision(case):
    """A = 0: D = bf16(beta * C) with beta a power of two, so the product is
    exact in fp32 and the one rounding is the oracle's."""
    M, N, K, split, packed = case
    p = f32_problem(M, N, K, seed=0xC0DE + M + N)
    p["A"][:] = 0
    d = gemm_gpu(p, split_k=split, b_packed=packed)
    _, _, dref = oracle_ref(p)
    assert np.array_equal(d, dref), "%d of %d elements differ" % (int((d != dref).sum()), d.size)


def test_kernel_families_covered():
    kinds = {mx.mxgemm_plan(M, N, K, int(pk), s, 256)["kernel"] for M, N, K, s, pk in F32_CASES}
    assert kinds == {0, 1, 2}


def _err_frac(d_bits, ref):
    d = bf16_to_f64(d_bits)
    return float(np.abs(d - ref).max() / np.abs(ref).max())


def test_bf16_atomic_split_error_against_the_pages_table():
    M, N, K = 256, 1024, 4096
    p = inputs.make_problem(M, N, K, seed=0xA70, e=(124, 130), beta=0.0)  # exponents 2^-3 .. 2^3
    say("case bf16-atomic split-K, oracle reference")
    ref, mag, _ = oracle_ref(p)
    rows = []
    for s in (1, 2, 4, 8, 16):
        assert mx.mxgemm_plan(M, N, K, 0, s, 256)["split_k"] == s
        d32 = gemm_gpu(p, split_k=s)
        dat = gemm_gpu(p, split_k=s, split_mode=mx.SPLIT_BF16_ATOMIC)
        assert_parity(d32, ref, mag, "fp32 split %d" % s)
        e32, eat = _err_frac(d32, ref), _err_frac(dat, ref)
        rows.append((s, e32, eat))
        say("split %2d: fp32 partials %.3f %%, bf16 atomics %.3f %% (pages: %.2f %%)"
            % (s, 100 * e32, 100 * eat, PAGE_SPLIT_ERR[s]))
        assert eat <= PAGE_BOUND, "bf16-atomic split %d: %.3f %% of max|ref|" % (s, 100 * eat)
        if s == 1:
            assert np.array_equal(d32, dat), "split 1 is the ordinary path in both modes"
    # the atomic reduction's error grows with the split; the fp32 one does not
    assert rows[-1][2] > rows[-1][1]
    assert max(r[1] for r in rows) <= 2 * rows[0][1] + 1e-12


def test_bf16_atomic_split_with_C_and_small_M():
    """beta != 0 (D starts at bf16(beta * C)) and M <= 64, which the atomic
    mode runs on the tiled kernel."""
    for M, N, K, s in ((32, 512, 4096, 4), (200, 300, 2048, 8)):
        p = inputs.make_problem(M, N, K, seed=0xA71 + M, e=(124, 130), beta=1.0, c_sigma=2.0)
        p["beta"] = 0.5
        dat = gemm_gpu(p, split_k=s, split_mode=mx.SPLIT_BF16_ATOMIC)
        ref, _, _ = oracle_ref(p)
        assert _err_frac(dat, ref) <= PAGE_BOUND

"""GPU parity of mxgemm_run_bf16a: the activation quantizer in front of the
GEMM (quantize-on-load at M = 1, the decode step), through the C-ABI.

The fused kernel quantizes with the quantizer's own block routine, so its D
must equal mxgemm_quantize followed by mxgemm_run on the same (skinny)
kernel bit for bit (same codes, same scales, same matrix instructions in the
same order; MXGEMM_GEMV=0 keeps the two-step path off the single-row GEMV,
whose K order differs); it is also checked
against the oracle's quantizer and GEMM.  Shapes cover the 1 x 8192 x 8192
decode, ragged N, a K tail (K % 128 != 0), forced split-K, packed B, C with
beta and float32 C, special values (NaN, +-inf, -0, zero blocks, exact
ties), and M > 1 (quantize into a library buffer, then the GEMM).
"""
import sys

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
import oracle
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxgpu import assert_parity, dev_bf16, dev_u8, host_bits, oracle_ref  # noqa: E402
from test_quantize import bf16_matrix  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def problem(M, N, K, seed, specials=False, beta=0.0, c_f32=False):
    rng = np.random.default_rng(seed)
    X = bf16_matrix(rng, M, K, spread=8.0, specials=specials)
    p = inputs.make_problem(M, N, K, seed=seed, e=(120, 134), beta=beta, c_sigma=2.0 if beta else None)
    if c_f32:
        p["C"] = (rng.standard_normal((M, N)) * 2.0).astype(np.float32)
    p["X"] = X
    p["alpha"] = 0.75
    if beta:
        p["beta"] = -0.5
    return p


def strides_for(p, packed):
    M, N, K = p["M"], p["N"], p["K"]
    c_f32 = p.get("C") is not None and p["C"].dtype == np.float32
    return mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, b_packed=int(packed),
                           c_f32=int(c_f32))


def device_operands(p, packed):
    M, N, K = p["M"], p["N"], p["K"]
    B, SB = dev_u8(p["B"]), dev_u8(p["SB"])
    if packed:
        info = mx.mxgemm_plan(M, N, K, 1, -1, 256)
        Bp = torch.empty(info["packed_b_bytes"], dtype=torch.uint8, device="cuda")
        SBp = torch.empty(info["packed_sb_bytes"], dtype=torch.uint8, device="cuda")
        mx.mxgemm_pack_b(Bp, SBp, B, SB, N, K)
        B, SB = Bp, SBp
    C = None
    if p.get("C") is not None and p["beta"] != 0.0:
        C = torch.from_numpy(p["C"]).cuda() if p["C"].dtype == np.float32 else dev_bf16(p["C"])
    return B, SB, C


def run_fused(p, packed=False, split=-1):
    M, N, K = p["M"], p["N"], p["K"]
    B, SB, C = device_operands(p, packed)
    X = dev_bf16(p["X"])
    D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mx.mxgemm_run_bf16a(D, C, X, B, SB, p["alpha"], p["beta"], M, N, K, strides=strides_for(p, packed),
                        split_k=split)
    torch.cuda.synchronize()
    return host_bits(D)


def run_two_step(p, packed=False, split=-1):
    M, N, K = p["M"], p["N"], p["K"]
    B, SB, C = device_operands(p, packed)
    X = dev_bf16(p["X"])
    A = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    SA = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    mx.mxgemm_quantize(A, SA, X, M, K)
    D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mx.mxgemm_run(D, C, A, B, SA, SB, p["alpha"], p["beta"], M, N, K, strides=strides_for(p, packed),
                  split_k=split)
    torch.cuda.synchronize()
    return host_bits(D)


def same_bits(a, b):
    return np.array_equal(a, b)


# (N, K, packed, split, beta, c_f32)
DECODE = [
    (8192, 8192, False, -1, 0.0, False),
    (8192, 8192, True, -1, 0.0, False),
    (1000, 2048, False, -1, 1.0, False),
    (777, 1056, False, -1, 1.0, True),    # K tail
    (64, 8192, False, 16, 0.0, False),    # forced split
    (300, 4096, True, 4, 1.0, False),
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "1x%dx%d%s_s%d%s" % (
    c[0], c[1], "_packed" if c[2] else "", c[3], "_c32" if c[5] else ("_c" if c[4] else "")))
def test_fused_decode_matches_quantize_then_gemm(case, monkeypatch):
    N, K, packed, split, beta, c_f32 = case
    # the two-step path on the skinny kernel (it would run the single-row
    # GEMV at 1 x 8192 x 8192, whose K order differs; tests/test_gemv.py)
    monkeypatch.setenv("MXGEMM_GEMV", "0")
    p = problem(1, N, K, seed=0xDEC0 + N + K, beta=beta, c_f32=c_f32)
    say("case fused decode", case)
    d = run_fused(p, packed, split)
    d2 = run_two_step(p, packed, split)
    assert same_bits(d, d2), "%d of %d elements differ" % (int((d != d2).sum()), d.size)
    # and against the oracle's quantizer and GEMM
    p["A"], p["SA"] = oracle.quantize_mxfp4(p["X"])
    cols = None if N * K <= 4 * 2 ** 20 else np.sort(np.random.default_rng(N).choice(N, 256, replace=False))
    ref, mag, _ = oracle_ref(p, cols=cols)
    assert_parity(d if cols is None else d[:, cols], ref, mag, "fused decode %s" % (case,))


def test_fused_decode_special_values():
    """NaN / inf blocks (scale 0xFF), -0, zero blocks, exact ties, bf16
    subnormal blocks: the fused kernel matches the two-step path bit for
    bit and the oracle's quantizer and GEMM element by element.  With a NaN
    or infinity anywhere in the row, every output is NaN (a block of scale
    0xFF holds codes 0, and 0 x NaN is NaN); the same row with its NaN and
    infinities replaced by finite values checks the other specials against
    the oracle's values."""
    for K in (1024, 4096):
        p = problem(1, 512, K, seed=0x5BEC + K, specials=True)
        say("case fused decode specials K", K)
        d = run_fused(p)
        d2 = run_two_step(p)
        assert same_bits(d, d2)
        p["A"], p["SA"] = oracle.quantize_mxfp4(p["X"])
        assert (p["SA"] == 0xFF).any()
        ref, mag, _ = oracle_ref(p)
        assert np.isnan(ref).all()
        assert_parity(d, ref, mag, "fused decode specials K=%d" % K)
        # finite specials only
        X = p["X"].copy()
        nonfinite = (X & 0x7F80) == 0x7F80
        X[nonfinite] = 0x3F80 | (X[nonfinite] & 0x8000)  # +-1.0
        p["X"] = X
        d = run_fused(p)
        assert same_bits(d, run_two_step(p))
        p["A"], p["SA"] = oracle.quantize_mxfp4(X)
        assert not (p["SA"] == 0xFF).any()
        ref, mag, _ = oracle_ref(p)
        assert np.isfinite(ref).all()
        assert_parity(d, ref, mag, "fused decode finite specials K=%d" % K)


@pytest.mark.parametrize("M", [2, 16, 40, 300])
def test_bf16a_several_rows_matches_quantize_then_gemm(M):
    N, K = 520, 2048
    p = problem(M, N, K, seed=0xB16A + M, beta=1.0)
    say("case bf16a rows", M)
    d = run_fused(p)
    d2 = run_two_step(p)
    assert same_bits(d, d2)


@pytest.mark.parametrize("nr", [2, 4])
def test_fused_decode_wider_row_groups(nr, monkeypatch):
    """32 and 64 rows of B per workgroup (MXGEMM_FORCE_NR; the planner picks
    16 at M = 1): the quantize-on-load kernels for those row groups, row-major
    and packed B, against the two-step path."""
    monkeypatch.setenv("MXGEMM_FORCE_NR", str(nr))
    assert mx.mxgemm_plan(1, 1000, 2048, 0, -1, 256)["tile_n"] == 16 * nr
    for packed in (False, True):
        p = problem(1, 1000, 2048, seed=0x4E52 + nr, beta=1.0)
        say("case fused decode nr", nr, "packed", packed)
        d = run_fused(p, packed)
        d2 = run_two_step(p, packed)
        assert same_bits(d, d2)

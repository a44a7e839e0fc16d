"""GPU parity of the GEMV (`gemv_m1_n4`: M == 1; `gemv_m4_n4` and
`gemv_m8_n4`: 2 <= M <= 8 with FP4 A; row-major FP4 B, K a multiple of 2048), through the C-ABI,
against the oracle.

The planner sends M == 1 with a row-major B (A in FP4, FP8, BF8 or either
FP6) to this kernel when K % 2048 == 0
and its 4-row workgroups give every compute unit one (N >= 4 x CUs);
MXGEMM_GEMV=0 keeps such shapes on the skinny kernel.  Cases: one chunk per
wave (K = 2048, 6144 -- one wave idle -- and 8192), several chunks per wave
(K = 16384, 28672 and 2^18: the two-register-set loop, waves with unequal
chunk counts), ragged N (a last workgroup with 1, 2 or 3 rows), beta with bf16
and float32 C, D aliasing C, padded rows of every operand, the E8M0
special scale codes, and quantize-then-GEMM beside the fused bf16-A
decode (which stays on the skinny kernel).  Source of the operation:
asm_f4gemm README, problem statement and "Data layouts".
"""
import sys

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
import oracle
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxgpu import assert_parity, dev_bf16, dev_u8, gemm_gpu, host_bits, oracle_ref  # noqa: E402
from test_decode import problem, run_fused, run_two_step  # noqa: E402
from test_specials import with_special_scales  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def lib_loaded():
    mx.lib()
    yield
    mx.mxgemm_release_workspaces()


def planned(M, N, K, b_packed=0, split=-1):
    return mx.mxgemm_query(M, N, K, b_packed, split)["kernel_name"]


# (N, K): chunks per wave 1 (K <= 8192) or several; N % 4 = 0..3
SHAPES = [(1024, 2048), (1027, 6144), (8192, 8192), (2050, 16384), (1025, 28672), (8193, 2048)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "1x%dx%d" % s)
@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_gemv_matches_oracle(shape, beta):
    N, K = shape
    assert planned(1, N, K) == "gemv_m1_n4"
    p = inputs.make_problem(1, N, K, seed=0x6E00 + N + K, e=(120, 134), beta=beta, c_sigma=2.0 if beta else None)
    p["alpha"] = 0.5
    if beta:
        p["beta"] = -0.75
    say("case gemv", shape, "beta", beta)
    d = gemm_gpu(p)
    ref, mag, _ = oracle_ref(p)
    assert_parity(d, ref, mag, "gemv %s beta=%g" % (shape, beta))


FORMATS = {1: "e4m3", 2: "e5m2", 3: "e2m3", 4: "e3m2"}


@pytest.mark.parametrize("fmt", list(FORMATS), ids=lambda f: FORMATS[f])
@pytest.mark.parametrize("shape", [(1027, 6144), (2050, 16384)], ids=lambda s: "1x%dx%d" % s)
def test_gemv_wider_A_matches_oracle(shape, fmt):
    """A in FP8 E4M3, BF8 E5M2, FP6 E2M3 or FP6 E3M2 ("CDNA4 dense MFMA
    builtins", "Mixed-precision with scaling"), B FP4, on the GEMV: one chunk
    per wave and the two-set loop, ragged N, C with beta."""
    N, K = shape
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, a_format=fmt)
    assert mx.mxgemm_query_ex(1, N, K, st, -1)["kernel_name"] == "gemv_m1_n4"
    e = (120, 134) if fmt in (3, 4) else (110, 130)
    p = inputs.make_problem(1, N, K, seed=0x6EF0 + 31 * fmt + N, e=e, beta=1.0, c_sigma=2.0, a_fmt=fmt)
    p["alpha"], p["beta"] = 0.5, -0.75
    say("case gemv", FORMATS[fmt], shape)
    ref, mag, _ = oracle_ref(p)
    assert_parity(gemm_gpu(p), ref, mag, "gemv %s %s" % (FORMATS[fmt], shape))


def test_gemv_long_K():
    """K = 2^18 (128 chunks, 32 per wave through the two-set loop; 128 MiB
    of B): against the oracle element by element."""
    N, K = 1024, 1 << 18
    assert planned(1, N, K) == "gemv_m1_n4"
    p = inputs.make_problem(1, N, K, seed=0x6E18, e=(120, 134))
    say("case gemv long K", (1, N, K))
    d = gemm_gpu(p)
    ref, mag, _ = oracle_ref(p)
    assert_parity(d, ref, mag, "gemv long K")


@pytest.mark.parametrize("M", [2, 3, 4, 5, 7, 8])
@pytest.mark.parametrize("shape", [(1024, 2048), (1027, 6144), (2050, 16384)], ids=lambda s: "x%dx%d" % s)
def test_gemv_small_batch_matches_oracle(shape, M, monkeypatch):
    """2 <= M <= 8 (FP4 A): A rows through the B-like operand lanes, one
    accumulator per group of 4 A rows; padded A and scale rows (pitches beyond K), C with
    beta; against the oracle, and the skinny kernel (MXGEMM_GEMV=0) on the
    same problem within the same tolerance."""
    N, K = shape
    kname = "gemv_m4_n4" if M <= 4 else "gemv_m8_n4"
    assert planned(M, N, K) == kname
    p = inputs.make_problem(M, N, K, seed=0x6E40 + 17 * M + N, e=(118, 136), beta=1.0, c_sigma=2.0)
    p["alpha"], p["beta"] = 0.5, -0.75
    ref, mag, _ = oracle_ref(p)
    lda, ldsa = K + 128, K // 32 + 16
    Apad = np.zeros((M, lda // 2), dtype=np.uint8)
    Apad[:, : K // 2] = p["A"]
    SApad = np.full((M, ldsa), 0xFF, dtype=np.uint8)  # NaN scale bytes past each row's K
    SApad[:, : K // 32] = p["SA"]
    A, SA, B, SB = dev_u8(Apad), dev_u8(SApad), dev_u8(p["B"]), dev_u8(p["SB"])
    C = dev_bf16(p["C"])
    st = mx.make_strides(ldd=N, ldc=N, lda=lda, ldb=K, ldsa=ldsa, ldsb=K // 32)
    assert mx.mxgemm_query_ex(M, N, K, st, -1)["kernel_name"] == kname
    say("case gemv small batch", (M, N, K))
    D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mx.mxgemm_run(D, C, A, B, SA, SB, p["alpha"], p["beta"], M, N, K, strides=st)
    torch.cuda.synchronize()
    assert_parity(host_bits(D), ref, mag, "gemv M=%d %s" % (M, shape))
    monkeypatch.setenv("MXGEMM_GEMV", "0")
    assert planned(M, N, K).startswith("skinny")
    assert_parity(gemm_gpu(p), ref, mag, "skinny M=%d %s" % (M, shape))


def test_gemv_f32_C_and_in_place():
    N, K = 1030, 8192
    p = inputs.make_problem(1, N, K, seed=0x6EF3, beta=1.0, c_sigma=2.0)
    p["C"] = (np.random.default_rng(3).standard_normal((1, N)) * 2.0).astype(np.float32)
    say("case gemv f32 C")
    assert_parity(gemm_gpu(p), *oracle_ref(p)[:2], "gemv f32 C")
    # D aliasing a bf16 C
    p = inputs.make_problem(1, N, K, seed=0x6EA1, beta=1.0, c_sigma=2.0)
    p["alpha"], p["beta"] = 2.0, -1.0
    ref, mag, _ = oracle_ref(p)
    A, B, SA, SB = dev_u8(p["A"]), dev_u8(p["B"]), dev_u8(p["SA"]), dev_u8(p["SB"])
    CD = dev_bf16(p["C"])
    say("case gemv in place")
    mx.mxgemm_run(CD, CD, A, B, SA, SB, 2.0, -1.0, 1, N, K)
    torch.cuda.synchronize()
    assert_parity(host_bits(CD), ref, mag, "gemv in place")


def test_gemv_padded_rows():
    """B rows, scale rows and D with pitches beyond their lengths (B pitch a
    multiple of 32 elements, scale pitches multiples of 16 bytes: the GEMV's
    requirements)."""
    N, K = 1100, 4096
    ldb, ldsb, ldd = K + 64, K // 32 + 16, N + 6
    p = inputs.make_problem(1, N, K, seed=0x6EBD, e=(118, 136))
    ref, mag, _ = oracle_ref(p)
    Bpad = np.zeros((N, ldb // 2), dtype=np.uint8)
    Bpad[:, : K // 2] = p["B"]
    SBpad = np.full((N, ldsb), 0xFF, dtype=np.uint8)  # NaN scale bytes past each row's K
    SBpad[:, : K // 32] = p["SB"]
    A, SA = dev_u8(p["A"]), dev_u8(p["SA"])
    B, SB = dev_u8(Bpad), dev_u8(SBpad)
    D = torch.full((1, ldd), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = mx.make_strides(ldd=ldd, ldc=ldd, lda=K, ldb=ldb, ldsa=K // 32, ldsb=ldsb)
    assert mx.mxgemm_query_ex(1, N, K, st, -1)["kernel_name"] == "gemv_m1_n4"
    say("case gemv padded")
    mx.mxgemm_run(D, None, A, B, SA, SB, p["alpha"], 0.0, 1, N, K, strides=st)
    torch.cuda.synchronize()
    bits = host_bits(D)
    assert_parity(bits[:, :N], ref, mag, "gemv padded")
    assert (bits[:, N:] == host_bits(torch.full((1, ldd - N), float("nan"), dtype=torch.bfloat16))).all()


def test_gemv_special_scale_codes():
    """About 2 % of the scale bytes of A and B replaced by 0x00, 0x01, 0xFE
    or 0xFF (A: not 0xFF, which would make every output NaN)."""
    N, K = 1040, 6144
    p = with_special_scales(inputs.make_problem(1, N, K, seed=0x6E5C, e=(118, 136)), seed=0x6E5C)
    p["SA"][p["SA"] == 0xFF] = 0xFE
    ref, mag, _ = oracle_ref(p)
    say("case gemv special scales")
    assert planned(1, N, K) == "gemv_m1_n4"
    assert_parity(gemm_gpu(p), ref, mag, "gemv special scales")
    assert np.isnan(ref).any() and (np.abs(ref) > 2.0 ** 128).any()


def test_gemv_and_skinny_agree(monkeypatch):
    """The same problem on the skinny kernel (MXGEMM_GEMV=0): both within the
    oracle's tolerance; their K orders differ, so bits may differ."""
    N, K = 4096, 16384
    p = inputs.make_problem(1, N, K, seed=0x6E6E, e=(120, 134))
    ref, mag, _ = oracle_ref(p)
    d_gemv = gemm_gpu(p)
    monkeypatch.setenv("MXGEMM_GEMV", "0")
    assert planned(1, N, K).startswith("skinny")
    d_skinny = gemm_gpu(p)
    assert_parity(d_gemv, ref, mag, "gemv")
    assert_parity(d_skinny, ref, mag, "skinny")


def test_gemv_plan_conditions():
    """Only M == 1, row-major B, K % 2048 == 0, unsplit, N >= 4 x CUs."""
    ncu = mx.mxgemm_query(1, 8192, 8192)["num_cu"]
    assert planned(1, 4 * ncu, 2048) == "gemv_m1_n4"
    assert planned(1, 4 * ncu - 4, 2048) != "gemv_m1_n4"
    assert planned(1, 8192, 8192, b_packed=1) != "gemv_m1_n4"
    assert planned(1, 8192, 8192 + 1024) != "gemv_m1_n4"
    assert planned(2, 8192, 8192) == "gemv_m4_n4"
    assert planned(8, 8192, 8192) == "gemv_m8_n4"
    assert planned(9, 8192, 8192).startswith("skinny")
    assert planned(1, 8192, 8192, split=2) != "gemv_m1_n4"
    assert planned(1, 8192, 8192, split=1) == "gemv_m1_n4"


def test_fused_decode_beside_the_gemv(monkeypatch):
    """The fused bf16-A decode (mxgemm_run_bf16a) stays on the skinny
    kernel's quantize-on-load; quantize-then-GEMM at the same shape runs the
    GEMV.  Both match the oracle's quantizer and GEMM; with the GEMV switched
    off the two paths are bit-identical."""
    N, K = 8192, 8192
    p = problem(1, N, K, seed=0x6ED0, beta=1.0)
    say("case fused decode beside the gemv")
    d = run_fused(p)
    d_gemv = run_two_step(p)
    p["A"], p["SA"] = oracle.quantize_mxfp4(p["X"])
    ref, mag, _ = oracle_ref(p)
    assert_parity(d, ref, mag, "fused decode")
    assert_parity(d_gemv, ref, mag, "quantize then gemv")
    monkeypatch.setenv("MXGEMM_GEMV", "0")
    assert np.array_equal(d, run_two_step(p))

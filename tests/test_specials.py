"""GPU parity on the special values of the operand formats, against the oracle.

The E8M0 scale codes at the ends of the range -- 0x00 (2^-127 by reading S1
of the pages' formula 2^(e-127)), 0x01, 0xFE (2^127) and 0xFF (NaN) -- and
the FP8 NaN / infinity codes of a wider A run through every kernel family
(M = 1 and M <= 16: skinny; 16 < M <= 64: rows; M > 64: tiled two-stage,
four-slot ring and persistent 256 x 256; FP6 A on the dense FP6 tile and
the 8-bit tile), row-major, packed B and packed B with packed A scales,
unsplit and split K, and are compared element by
element with the oracle under the rules of tests/mxgpu.py (NaN must match
NaN, infinities must match the oracle's bf16 rounding, bf16 subnormals are
compared with an absolute half-spacing, and the fp32 accumulation's own
overflow is allowed only where the sum of |products| reaches the fp32
range).  Sources: asm_f4gemm README, "Data layouts" / "A_scale / B_scale"
(E8M0 value 2^(e-127), 0xFF NaN); "CDNA4 dense MFMA builtins",
"Mixed-precision with scaling" (FP8 inputs, fp32 accumulation).
"""
import sys

import numpy as np
import pytest

import block_scaled_precision_mxfp4_amd as mx
from block_scaled_precision_mxfp4_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxgpu import FP32_OVERFLOW, assert_parity, gemm_gpu, oracle_ref  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def lib_loaded():
    mx.lib()
    yield
    mx.mxgemm_release_workspaces()


PACK_MODES = [(False, False), (True, False), (True, True)]
SPECIAL_CODES = np.array([0x00, 0x01, 0xFE, 0xFF], dtype=np.uint8)

# skinny M = 1, skinny M <= 16, rows, tiled (planner's pick), tiled 256-row tiles
SHAPES = [(1, 520, 2048), (8, 520, 2048), (40, 520, 4096), (300, 520, 2048), (256, 1024, 1024)]


def with_special_scales(p, seed, prob=0.02):
    """Replace a fraction of both scale matrices' bytes by the special codes."""
    rng = np.random.default_rng(seed)
    for key in ("SA", "SB"):
        S = p[key].copy()
        mask = rng.random(S.shape) < prob
        S[mask] = rng.choice(SPECIAL_CODES, int(mask.sum()))
        p[key] = S
    return p


def run_modes(p, what, splits=(1, 4), check=None):
    ref, mag, _ = oracle_ref(p)
    for packed, sa_packed in PACK_MODES:
        for s in splits:
            say("case", what, "packed", packed, sa_packed, "split", s)
            d = gemm_gpu(p, split_k=s, b_packed=packed, sa_packed=sa_packed)
            assert_parity(d, ref, mag, "%s packed=%s,%s split=%d" % (what, packed, sa_packed, s))
            if check is not None:
                check(d)
    return ref, mag


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_special_scale_codes(shape):
    """About 2 % of the scale bytes of A and B replaced by 0x00, 0x01, 0xFE or
    0xFF among normal exponents 118..136: NaN rows and columns, overflowing
    blocks and vanishing blocks mixed with ordinary ones."""
    M, N, K = shape
    p = with_special_scales(inputs.make_problem(M, N, K, seed=0x5C + M, e=(118, 136)), seed=0x5C + M)
    if M == 1:  # one NaN scale in the only row of A would make every output NaN
        p["SA"][p["SA"] == 0xFF] = 0xFE
    ref, _ = run_modes(p, "special scales %dx%dx%d" % shape)
    assert np.isnan(ref).any() and (np.abs(ref) > 2.0 ** 128).any(), "the case must hold NaN and overflowing outputs"


@pytest.mark.parametrize("tile", [0, 1, 2, 3])
def test_special_scale_codes_every_tile(tile, monkeypatch):
    """The same mixture on each tile shape, two-stage and four-slot ring."""
    monkeypatch.setenv("MXGEMM_FORCE_TILE", str(tile))
    M, N, K = 300, 520, 2048
    p = with_special_scales(inputs.make_problem(M, N, K, seed=0x7E + tile, e=(118, 136)), seed=0x7E + tile)
    ref, mag, _ = oracle_ref(p)
    for pipe in ("two-stage", "deep"):
        monkeypatch.setenv("MXGEMM_TILE_PIPELINE", pipe)
        for packed, sa_packed in PACK_MODES:
            say("case special scales tile", tile, pipe, "packed", packed, sa_packed)
            d = gemm_gpu(p, split_k=2, b_packed=packed, sa_packed=sa_packed)
            assert_parity(d, ref, mag, "tile %d %s packed=%s,%s" % (tile, pipe, packed, sa_packed))


def test_special_scale_codes_persistent():
    """The persistent 256 x 256 form (fully packed, 400 tiles on the compute
    units, beta = 0): every column of sampled rows, special rows included."""
    M, N, K = 5120, 5120, 1024
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, b_packed=1, sa_packed=1)
    info = mx.mxgemm_query_ex(M, N, K, st, -1)
    assert info["persist_grid"] > 0, info
    p = with_special_scales(inputs.make_problem(M, N, K, seed=0x9E, e=(118, 136)), seed=0x9E, prob=0.002)
    say("case special scales persistent", (M, N, K), info["kernel_name"])
    d = gemm_gpu(p, split_k=-1, b_packed=True, sa_packed=True)
    special_rows = np.nonzero((p["SA"] == 0xFF).any(axis=1) | (p["SA"] == 0xFE).any(axis=1))[0][:24]
    rows = np.unique(np.concatenate([special_rows, np.arange(0, M, 97), [M - 1]])).astype(np.int64)
    ref, mag, _ = oracle_ref(p, rows=rows)
    assert np.isnan(ref).any() and (np.abs(ref) > 2.0 ** 128).any()
    assert_parity(d[rows], ref, mag, "persistent special scales")


@pytest.mark.parametrize("tile", ["tile_fp6_256x256", "tile_a8_128x256"])
def test_special_scale_codes_fp6_tiles(tile, monkeypatch):
    """The same mixture with FP6 E2M3 A on the dense FP6 tile (its A scales
    shuffled by the re-layout and held in registers) and on the 8-bit tile
    (the padded copy), row-major and packed B, unsplit and split K."""
    monkeypatch.setenv("MXGEMM_A8_TILE", tile)
    M, N, K = 300, 520, 2048
    fmt = mx.FMT_FP6_E2M3
    p = with_special_scales(inputs.make_problem(M, N, K, seed=0xF6 + len(tile), e=(118, 136), a_fmt=fmt),
                            seed=0xF6 + len(tile))
    ref, mag, _ = oracle_ref(p)
    assert np.isnan(ref).any() and (np.abs(ref) > 2.0 ** 128).any()
    for packed in (False, True):
        st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, b_packed=int(packed), a_format=fmt)
        assert mx.mxgemm_plan_ex(M, N, K, st, 1, 256)["kernel_name"] == tile
        for s in (1, 2):
            say("case special scales fp6", tile, "packed", packed, "split", s)
            d = gemm_gpu(p, split_k=s, b_packed=packed)
            assert_parity(d, ref, mag, "fp6 %s packed=%s split=%d" % (tile, packed, s))


@pytest.mark.parametrize("shape", SHAPES[:4], ids=lambda s: "%dx%dx%d" % s)
def test_extreme_scale_pairs_are_exact(shape):
    """Each K block's scale pair sums near 254 -- (0xFE, 0x00), (0xFE, 0x01),
    (0x00, 0xFE), (0x01, 0xFE), (0x01, 0xFD), (0xFD, 0x02), (0x00, 0xFE) or
    (127, 127) -- so every product is finite: the result must be the ordinary
    tolerance everywhere, which pins 0x00 at 2^-127 and 0xFE at 2^127 on the
    hardware (0x00 read as 2^-126 would double those blocks)."""
    M, N, K = shape
    p = inputs.make_problem(M, N, K, seed=0x9A + M, e=(124, 130))
    rng = np.random.default_rng(0x9A + M)
    pairs = np.array([(0xFE, 0x00), (0xFE, 0x01), (0x00, 0xFE), (0x01, 0xFE), (0x01, 0xFD), (0xFD, 0x02),
                      (127, 127), (0x00, 0xFE)], dtype=np.uint8)
    ch = pairs[rng.integers(0, len(pairs), K // 32)]
    p["SA"] = np.tile(ch[:, 0], (M, 1)).copy()
    p["SB"] = np.tile(ch[:, 1], (N, 1)).copy()
    ref, mag = run_modes(p, "extreme pairs %dx%dx%d" % shape)
    assert np.isfinite(ref).all() and (mag < FP32_OVERFLOW).all()


@pytest.mark.parametrize("shape", [(1, 64, 1024), (8, 64, 1024), (40, 64, 1024), (300, 64, 1024)],
                         ids=lambda s: "%dx%dx%d" % s)
@pytest.mark.parametrize("base", [124, 116, 107])
def test_subnormal_range_outputs(shape, base):
    """Scale pairs summing to base-1 .. base+3 (A scales 0..2): products from
    about 2^-128 down to 2^-150, i.e. results in and below bf16's subnormal
    range, where the output rounding is absolute."""
    M, N, K = shape
    p = inputs.make_problem(M, N, K, seed=0x71 + base + M, e=(124, 130))
    rng = np.random.default_rng(0x71 + base + M)
    p["SA"] = rng.integers(0, 3, (M, K // 32)).astype(np.uint8)
    p["SB"] = (base - 1 + rng.integers(0, 3, (N, K // 32))).astype(np.uint8)
    ref, _ = run_modes(p, "subnormal base %d %dx%dx%d" % ((base,) + shape))
    tiny = np.abs(ref) < 2.0 ** -126
    assert tiny.all() if base <= 107 else (tiny.any() if base <= 116 else True)


def test_nan_scale_on_zero_codes():
    """A NaN scale (0xFF) whose 32 codes are all +-0 still makes every output
    of its row (A) or column (B) NaN, as 0 x NaN is NaN in the oracle; a
    zero-code block under an ordinary scale contributes nothing."""
    for M, N, K in [(1, 300, 1024), (8, 300, 1024), (40, 300, 1024), (300, 300, 1024)]:
        p = inputs.make_problem(M, N, K, seed=0x2E0 + M, e=(120, 134))
        A, SA, B, SB = p["A"].copy(), p["SA"].copy(), p["B"].copy(), p["SB"].copy()
        ra, kb = M // 2, 5
        A[ra, kb * 16:(kb + 1) * 16] = 0x80  # +0 and -0 codes
        SA[ra, kb] = 0xFF
        cb, kb2 = 17, 9
        B[cb, kb2 * 16:(kb2 + 1) * 16] = 0x08
        SB[cb, kb2] = 0xFF
        B[cb + 1, kb2 * 16:(kb2 + 1) * 16] = 0x00  # zero block, ordinary scale
        p.update(A=A, SA=SA, B=B, SB=SB)
        ref, _ = run_modes(p, "nan on zero codes M=%d" % M)
        assert np.isnan(ref[ra]).all() and np.isnan(ref[:, cb]).all()


def test_overflow_to_infinity():
    """Blocks under scale pairs (0xFE, 0xFE) with codes of one sign: every
    partial sum of the affected outputs overflows in the same direction, so
    the GPU must give the infinity of that sign that the oracle's bf16
    rounding gives."""
    for M, N, K in [(1, 300, 1024), (8, 300, 1024), (40, 300, 1024), (300, 300, 1024)]:
        p = inputs.make_problem(M, N, K, seed=0x1F0 + M, e=(120, 134))
        A, SA, B, SB = p["A"].copy(), p["SA"].copy(), p["B"].copy(), p["SB"].copy()
        kb = 3
        rows = np.arange(0, M, 3)
        A[rows, kb * 16:(kb + 1) * 16] = 0x77                            # +6
        A[rows[1::2], kb * 16:(kb + 1) * 16] = 0xFF                      # -6
        SA[rows, kb] = 0xFE
        cols = np.arange(0, N, 5)
        B[cols, kb * 16:(kb + 1) * 16] = 0x77
        SB[cols, kb] = 0xFE
        p.update(A=A, SA=SA, B=B, SB=SB)
        # the designed block: +inf in rows with +6 codes, -inf in rows with -6
        want = np.where(np.isin(rows, rows[1::2]), 0xFF80, 0x7F80).astype(np.uint16)[:, None]

        def check(d):
            assert (d[np.ix_(rows, cols)] == want).all()

        ref, _ = run_modes(p, "overflow M=%d" % M, check=check)
        assert (np.abs(ref[np.ix_(rows, cols)]) > 2.0 ** 128).all()


@pytest.mark.parametrize("fmt", [1, 2], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("M", [1, 8, 40, 300])
def test_fp8_nan_and_inf_codes(fmt, M):
    """A in FP8 E4M3 (NaN codes 0x7F, 0xFF) or BF8 E5M2 (+-inf 0x7C, 0xFC and
    NaN 0x7D, 0xFE) mixed into otherwise finite codes: NaN and signed
    infinities must land where the oracle's fp64 sums put them (inf x 0 and
    inf - inf are NaN)."""
    N, K = 264, 1024
    p = inputs.make_problem(M, N, K, seed=0xF8 + M + fmt, e=(120, 134), a_fmt=fmt)
    A = p["A"].copy()
    rng = np.random.default_rng(M + fmt)
    mask = rng.random(A.shape) < (0.0005 if M > 1 else 0.002)
    codes = np.array([0x7F, 0xFF] if fmt == 1 else [0x7C, 0xFC, 0x7D, 0xFE], dtype=np.uint8)
    A[mask] = rng.choice(codes, int(mask.sum()))
    if M == 1:
        A[0, 10] = 0x7C if fmt == 2 else A[0, 10]  # a lone infinity at M = 1
    p["A"] = A
    ref, mag, _ = oracle_ref(p)
    for s in (1, 4):
        for packed in (False, True):
            say("case fp8 specials fmt", fmt, "M", M, "split", s, "packed", packed)
            d = gemm_gpu(p, split_k=s, b_packed=packed)
            assert_parity(d, ref, mag, "fp8 fmt %d M %d split %d packed %s" % (fmt, M, s, packed))
    assert np.isnan(ref).any()

"""Helpers for the GPU parity tests: device marshalling through the C-ABI
binding, and the element-wise comparison against the CPU oracle.

Tolerance (per element, floating point): |D - ref| <= 2^-7 |ref| + 2^-12 mag
+ 2^-133, with ref the exact fp64 value of alpha*A*B^T + beta*C and mag =
sum_k |a_ik b_jk|.  2^-7 |ref| covers the bf16 output rounding (at most 2^-8
relative, round to nearest) with a factor two to spare; 2^-12 mag covers
the fp32 accumulation inside the matrix instructions and the fp32 split-K
partial sums.  2^-133 is the bf16 output rounding below the normal range:
there bf16's spacing is the fixed 2^-133 (subnormals), so its rounding error
is absolute, at most 2^-134.  NaN must match NaN; +0 equals -0; an infinity
must match the oracle's rounding of ref to bf16 (+-inf beyond the largest
bf16).

One departure is inherent to the arithmetic: the matrix instructions and the
split-K reduction accumulate in fp32 ("CDNA4 dense MFMA builtins": fp32
results), so a partial sum beyond the fp32 range becomes +-inf (and +inf +
-inf gives NaN) even when the exact sum would come back into range.  Only an
element whose sum of |products| times max(1, |alpha|) reaches the fp32
overflow threshold can have such a partial sum (every partial sum is bounded
by it), and only there may the GPU give an infinity or NaN that the exact
value does not have, or an infinity of the other sign (that of the first
partial sum to overflow).
"""
from __future__ import annotations

import numpy as np
import torch

import block_scaled_precision_mxfp4_amd as mx
import oracle

TOL_REL = 2.0 ** -7
TOL_MAG = 2.0 ** -12
TOL_ABS = 2.0 ** -133
# fp32 round-to-nearest overflows at 2^128 - 2^103 (halfway to the next binade)
FP32_OVERFLOW = 2.0 ** 128 - 2.0 ** 103
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_gpu(p: dict, split_k: int = -1, b_packed: bool = False, D=None, stream=None, sa_packed: bool = False,
             split_mode: int = 0):
    """Run D = bf16(alpha A B^T + beta C) on the GPU for problem p (dense
    strides; b_packed: B and its scales pre-shuffled by mxgemm_pack_b;
    sa_packed: A's scales too, by mxgemm_pack_scales; a float32 p["C"] is
    passed as an f32 C).  With p["B_kn"] (MN-major codes [K, ldb/2], ldb =
    p["ldb_kn"]) B is passed MN-major and b_packed packs only its scales.
    Returns the bf16 bits of D as numpy uint16 [M, N]."""
    if p.get("B_kn") is not None:
        return gemm_gpu_kn(p, split_k, b_packed, sa_packed, D=D, stream=stream, split_mode=split_mode)
    M, N, K = p["M"], p["N"], p["K"]
    A, B, SA, SB = dev_u8(p["A"]), dev_u8(p["B"]), dev_u8(p["SA"]), dev_u8(p["SB"])
    c_f32 = p.get("C") is not None and p["C"].dtype == np.float32
    if p.get("C") is None:
        C = None
    elif c_f32:
        C = torch.from_numpy(np.ascontiguousarray(p["C"])).cuda()
    else:
        C = dev_bf16(p["C"])
    if D is None:
        D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    strides = None
    a_fmt = int(p.get("a_fmt", 0))
    if c_f32 or split_mode or a_fmt:
        strides = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32,
                                  c_f32=int(c_f32), split_mode=split_mode, a_format=a_fmt)
    if b_packed:
        info = mx.mxgemm_plan(M, N, K, 1, -1, 256)
        Bp = torch.empty(info["packed_b_bytes"], dtype=torch.uint8, device="cuda")
        SBp = torch.empty(info["packed_sb_bytes"], dtype=torch.uint8, device="cuda")
        mx.mxgemm_pack_b(Bp, SBp, B, SB, N, K)
        B, SB = Bp, SBp
        if sa_packed:
            SAp = torch.empty(info["packed_sa_bytes"], dtype=torch.uint8, device="cuda")
            mx.mxgemm_pack_scales(SAp, SA, M, K)
            SA = SAp
        strides = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=K, ldsa=K // 32, ldsb=K // 32, b_packed=1,
                                  sa_packed=int(sa_packed), c_f32=int(c_f32), split_mode=split_mode,
                                  a_format=a_fmt)
    mx.mxgemm_run(D, C if p["beta"] != 0.0 else None, A, B, SA, SB, p["alpha"], p["beta"], M, N, K,
                  strides=strides, split_k=split_k, stream=stream)
    torch.cuda.synchronize()
    return host_bits(D)


def gemm_gpu_kn(p: dict, split_k=-1, sb_packed=False, sa_packed=False, D=None, stream=None, split_mode=0):
    """gemm_gpu with B's codes MN-major (p["B_kn"], row pitch p["ldb_kn"]
    fp4 elements); sb_packed: scaleB shuffled by mxgemm_pack_scales."""
    M, N, K = p["M"], p["N"], p["K"]
    A, B, SA, SB = dev_u8(p["A"]), dev_u8(p["B_kn"]), dev_u8(p["SA"]), dev_u8(p["SB"])
    C = None
    if p.get("C") is not None:
        C = torch.from_numpy(np.ascontiguousarray(p["C"])).cuda() if p["C"].dtype == np.float32 else dev_bf16(p["C"])
    if D is None:
        D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    info = mx.mxgemm_plan(M, N, K, 1, -1, 256)
    if sb_packed:
        SBp = torch.empty(mx.mxgemm_plan(N, N, K, 1, -1, 256)["packed_sa_bytes"], dtype=torch.uint8, device="cuda")
        mx.mxgemm_pack_scales(SBp, SB, N, K)
        SB = SBp
    if sa_packed:
        SAp = torch.empty(info["packed_sa_bytes"], dtype=torch.uint8, device="cuda")
        mx.mxgemm_pack_scales(SAp, SA, M, K)
        SA = SAp
    c_f32 = p.get("C") is not None and p["C"].dtype == np.float32
    st = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=p["ldb_kn"], ldsa=K // 32, ldsb=K // 32, b_packed=int(sb_packed),
                         sa_packed=int(sa_packed), c_f32=int(c_f32), split_mode=split_mode, b_layout=mx.B_KN)
    mx.mxgemm_run(D, C if p["beta"] != 0.0 else None, A, B, SA, SB, p["alpha"], p["beta"], M, N, K,
                  strides=st, split_k=split_k, stream=stream)
    torch.cuda.synchronize()
    return host_bits(D)


def oracle_ref(p: dict, rows=None, cols=None):
    if p.get("B_kn") is not None:  # the oracle reads the same MN-major bytes
        return oracle.mxgemm(p["A"], p["SA"], p["B_kn"], p["SB"], p["K"], p["alpha"], p["beta"],
                             p.get("C"), rows=rows, cols=cols, a_fmt=int(p.get("a_fmt", 0)),
                             ldb=p["ldb_kn"], b_layout=1)
    return oracle.mxgemm(p["A"], p["SA"], p["B"], p["SB"], p["K"], p["alpha"], p["beta"],
                         p.get("C"), rows=rows, cols=cols, a_fmt=int(p.get("a_fmt", 0)))


def classify(d_bits: np.ndarray, ref: np.ndarray, mag: np.ndarray, alpha: float = 1.0):
    """Element-wise verdict (rules in the module docstring): returns (bad
    mask, excess over the bound where both values are finite, mask of
    those elements)."""
    d = bf16_to_f64(d_bits)
    ovf = mag * max(1.0, abs(alpha)) >= FP32_OVERFLOW  # a partial sum may leave the fp32 range
    nan_ref, nan_d = np.isnan(ref), np.isnan(d)
    # the oracle's own bf16 rounding gives +-inf beyond the largest bf16 (by
    # more than half a spacing)
    inf_ref = ~nan_ref & (np.abs(ref) >= BF16_MAX + 2.0 ** 119)
    inf_d = np.isinf(d)
    same_sign_inf = inf_d & (np.sign(d) == np.sign(ref))
    # a finite ref within the tolerance of the overflow threshold may round to inf
    near_top = np.abs(ref) + TOL_REL * np.abs(ref) + TOL_MAG * mag >= BF16_MAX + 2.0 ** 119
    bad = (nan_ref & ~nan_d) | (nan_d & ~nan_ref & ~ovf)
    # (with a possible fp32 overflow, the sign of the infinity is that of the
    # first partial sum to overflow, not necessarily that of the exact sum)
    bad |= inf_ref & ~nan_d & ~same_sign_inf & ~(ovf & inf_d)
    bad |= inf_d & ~inf_ref & ~nan_ref & ~ovf & ~(near_top & same_sign_inf)
    ok = ~(nan_ref | nan_d | inf_ref | inf_d)
    excess = np.full(ref.shape, -np.inf)
    with np.errstate(invalid="ignore", over="ignore"):
        excess[ok] = np.abs(d[ok] - ref[ok]) - (TOL_REL * np.abs(ref[ok]) + TOL_MAG * mag[ok] + TOL_ABS)
    bad |= ok & (excess > 0)
    return bad, excess, ok


def compare(d_bits: np.ndarray, ref: np.ndarray, mag: np.ndarray, alpha: float = 1.0):
    """Returns (n_bad, worst_excess, max_rel_err) for GPU bits vs the oracle
    (rules in the module docstring)."""
    bad, excess, ok = classify(d_bits, ref, mag, alpha)
    d = bf16_to_f64(d_bits)
    worst = float(excess[ok].max()) if ok.any() else 0.0
    nz = ok & (np.abs(ref) >= 2.0 ** -126)  # relative error over the normal range
    rel = float((np.abs(d[nz] - ref[nz]) / np.abs(ref[nz])).max()) if nz.any() else 0.0
    return int(np.count_nonzero(bad)), worst, rel


def assert_parity(d_bits, ref, mag, what="", alpha=1.0):
    n_bad, worst, rel = compare(d_bits, ref, mag, alpha)
    if n_bad:
        bad, _, _ = classify(d_bits, ref, mag, alpha)
        d = bf16_to_f64(d_bits)
        ex = ["(%s: ref %.6g mag %.6g gpu %.6g)" % (tuple(int(v) for v in ix), ref[tuple(ix)], mag[tuple(ix)],
                                                   d[tuple(ix)]) for ix in np.argwhere(bad)[:4]]
        raise AssertionError("%s: %d elements outside tolerance (worst excess %.3g, max rel %.3g) e.g. %s" % (
            what, n_bad, worst, rel, " ".join(ex)))
    return rel

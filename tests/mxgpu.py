"""Helpers for the GPU parity tests: device marshalling through the C-ABI
binding, and the element-wise comparison against the CPU oracle.

Tolerance (per element, floating point): |D - ref| <= 2^-7 |ref| + 2^-12 mag,
with ref the exact fp64 value of alpha*A*B^T + beta*C and mag = sum_k
|a_ik b_jk|.  2^-7 |ref| covers the bf16 output rounding (at most 2^-8
relative, round to nearest) with a factor two to spare; 2^-12 mag covers
the fp32 accumulation inside the matrix instructions and the fp32 split-K
partial sums.  NaN must match NaN; +0 equals -0.
"""
from __future__ import annotations

import numpy as np
import torch

import block_scaled_precision_mxfp4_amd as mx
import oracle

TOL_REL = 2.0 ** -7
TOL_MAG = 2.0 ** -12


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
    passed as an f32 C).  Returns the bf16 bits of D as numpy uint16 [M, N]."""
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


def oracle_ref(p: dict, rows=None, cols=None):
    return oracle.mxgemm(p["A"], p["SA"], p["B"], p["SB"], p["K"], p["alpha"], p["beta"],
                         p.get("C"), rows=rows, cols=cols, a_fmt=int(p.get("a_fmt", 0)))


def compare(d_bits: np.ndarray, ref: np.ndarray, mag: np.ndarray):
    """Returns (n_bad, worst_excess, max_rel_err) for GPU bits vs the oracle."""
    d = bf16_to_f64(d_bits)
    nan_ref, nan_d = np.isnan(ref), np.isnan(d)
    bad_nan = int(np.count_nonzero(nan_ref != nan_d))
    ok = ~(nan_ref | nan_d)
    err = np.abs(d[ok] - ref[ok])
    bound = TOL_REL * np.abs(ref[ok]) + TOL_MAG * mag[ok]
    excess = err - bound
    n_bad = int(np.count_nonzero(excess > 0)) + bad_nan
    worst = float(excess.max()) if excess.size else 0.0
    nz = np.abs(ref[ok]) > 0
    rel = float((err[nz] / np.abs(ref[ok][nz])).max()) if nz.any() else 0.0
    return n_bad, worst, rel


def assert_parity(d_bits, ref, mag, what=""):
    n_bad, worst, rel = compare(d_bits, ref, mag)
    assert n_bad == 0, "%s: %d elements outside tolerance (worst excess %.3g, max rel %.3g)" % (
        what, n_bad, worst, rel)
    return rel

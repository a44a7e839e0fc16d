"""Seeded synthetic inputs for the MXFP4 GEMM workloads.

This module only draws random bytes and values; it contains none of the
GEMM's arithmetic and is the one piece of code that the GPU path's callers
(tests, benchmark) and the CPU oracle's callers share.

Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; public-domain reference by S. Vigna), used
in its counter form: output i of a stream with seed s is mix(s + (i+1)*gamma).
Every tensor draws from its own stream (seed XOR a per-tensor tag), so the
shape of one tensor never shifts the values of another.

Storage formats follow the asm_f4gemm README ("Data layouts"):
  - A, B: row-major packed fp4x2 bytes [rows, K/2]; byte i holds element 2i
    in the low nibble and 2i+1 in the high nibble; codes are E2M1 nibbles.
  - SA, SB: E8M0 bytes [rows, K/32], one per 32 consecutive K elements.
  - C: bf16 [M, N] (stored here as uint16 bit patterns).
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
SEED_BASE = 0x4D5846500000

_TAGS = {"A": 0x41 << 40, "B": 0x42 << 40, "SA": 0x5341 << 40, "SB": 0x5342 << 40,
         "C": 0x43 << 40}

_CHUNK = 1 << 22  # draws per numpy batch (bounds temporary memory)


def splitmix64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """n consecutive SplitMix64 outputs (uint64) of stream `seed`, from index `start`."""
    out = np.empty(n, dtype=np.uint64)
    s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    with np.errstate(over="ignore"):
        for c0 in range(0, n, _CHUNK):
            c1 = min(n, c0 + _CHUNK)
            z = s + np.arange(start + c0 + 1, start + c1 + 1, dtype=np.uint64) * GAMMA
            z = (z ^ (z >> np.uint64(30))) * _M1
            z = (z ^ (z >> np.uint64(27))) * _M2
            out[c0:c1] = z ^ (z >> np.uint64(31))
    return out


def _stream(seed: int, tag: str) -> int:
    return (seed ^ _TAGS[tag]) & 0xFFFFFFFFFFFFFFFF


def _u32(seed: int, n: int) -> np.ndarray:
    """n uniform 32-bit draws (both halves of each 64-bit output)."""
    w = splitmix64(seed, (n + 1) // 2)
    return w.view(np.uint32)[:n]


def fp4_codes_packed(seed: int, rows: int, K: int, dist: str = "uniform") -> np.ndarray:
    """Packed fp4x2 matrix [rows, K/2] of E2M1 codes.

    dist = "uniform":   every nibble uniform over the 16 codes (a uniform
                        random byte is two independent uniform nibbles).
    dist = "half_zero": each nibble is 0x0 with probability 1/2, otherwise
                        uniform over 0x1..0xF (0x8, i.e. -0, included).
    """
    nbytes = rows * (K // 2)
    if dist == "uniform":
        w = splitmix64(seed, (nbytes + 7) // 8)
        return w.view(np.uint8)[:nbytes].reshape(rows, K // 2).copy()
    if dist == "half_zero":
        out = np.empty(nbytes, dtype=np.uint8)
        half = np.uint64(1 << 31)
        for b0 in range(0, nbytes, _CHUNK):
            b1 = min(nbytes, b0 + _CHUNK)
            # two 32-bit draws per byte: low nibble then high nibble
            w = splitmix64(seed, b1 - b0, start=b0).view(np.uint32).astype(np.uint64)
            nz = w >= half
            code = np.where(nz, np.uint64(1) + (((w - half) * np.uint64(15)) >> np.uint64(31)),
                            np.uint64(0)).astype(np.uint8)
            out[b0:b1] = code[0::2] | (code[1::2] << np.uint8(4))
        return out.reshape(rows, K // 2)
    raise ValueError("unknown code distribution %r" % dist)


# A formats besides FP4 (the library's ids): element width in bits
FORMAT_BITS = {0: 4, 1: 8, 2: 8, 3: 6, 4: 6}


def wide_codes(seed: int, rows: int, K: int, fmt: int) -> np.ndarray:
    """A matrix of format fmt (1 FP8 E4M3, 2 BF8 E5M2, 3 FP6 E2M3, 4 FP6
    E3M2) as row-major bytes [rows, K * w / 8]: a little-endian bit stream
    of w-bit codes per row (element k at bits k*w .. k*w+w-1).  Codes are
    uniform over the format's finite values: E4M3 leaves out its two NaN
    codes (exponent and mantissa all ones), E5M2 its eight infinity and NaN
    codes (exponent all ones); the FP6 formats have none."""
    n = rows * K
    h = _u32(seed, n).astype(np.uint64)
    if fmt in (3, 4):
        codes = (h >> np.uint64(26)).astype(np.uint32).reshape(rows, K // 4, 4)  # 6 bits
        v = codes[..., 0] | (codes[..., 1] << 6) | (codes[..., 2] << 12) | (codes[..., 3] << 18)
        out = np.empty((rows, K // 4, 3), dtype=np.uint8)
        out[..., 0], out[..., 1], out[..., 2] = v & 0xFF, (v >> 8) & 0xFF, (v >> 16) & 0xFF
        return out.reshape(rows, K * 3 // 4)
    if fmt == 1:
        finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    elif fmt == 2:
        finite = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], dtype=np.uint8)
    else:
        raise ValueError("unknown A format %r" % fmt)
    idx = (h * np.uint64(len(finite))) >> np.uint64(32)
    return finite[idx.astype(np.int64)].reshape(rows, K)


def to_mn_major(B: np.ndarray, N: int, K: int, ldb: int, pad: int = 0) -> np.ndarray:
    """Re-store a K-major packed fp4x2 B [N, K/2] as MN-major [K, ldb/2]
    bytes: row k holds the codes of columns 0..N-1 at that k (element n in
    the low nibble of byte n/2 when n is even), columns N..ldb-1 hold the
    nibble `pad`.  A pure data movement of the codes."""
    codes = np.empty((N, K), dtype=np.uint8)
    codes[:, 0::2] = B[:, : K // 2] & 0x0F
    codes[:, 1::2] = B[:, : K // 2] >> 4
    kn = np.full((K, ldb), pad & 0xF, dtype=np.uint8)
    kn[:, :N] = codes.T
    return (kn[:, 0::2] | (kn[:, 1::2] << 4)).astype(np.uint8)


def e8m0_scales(seed: int, rows: int, K: int, lo: int, hi: int) -> np.ndarray:
    """E8M0 bytes [rows, K/32], exponents uniform over lo..hi inclusive."""
    n = rows * (K // 32)
    span = np.uint64(hi - lo + 1)
    h = _u32(seed, n).astype(np.uint64)
    e = np.uint64(lo) + ((h * span) >> np.uint64(32))
    return e.astype(np.uint8).reshape(rows, K // 32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (input preparation)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    r = r.astype(np.uint16)
    r[nan] = np.uint16(0x7FC0)
    return r


def gaussian_bf16(seed: int, rows: int, cols: int, sigma: float) -> np.ndarray:
    """bf16 bit patterns [rows, cols] of N(0, sigma^2) draws (Box-Muller)."""
    n = rows * cols
    w = splitmix64(seed, 2 * n)
    u1 = ((w[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = (w[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2) * sigma
    return f32_to_bf16_bits(z.astype(np.float32)).reshape(rows, cols)


def gaussian_f16(seed: int, rows: int, cols: int, sigma: float) -> np.ndarray:
    """fp16 bit patterns [rows, cols] of N(0, sigma^2) draws (Box-Muller,
    rounded to nearest by numpy's float16 conversion)."""
    n = rows * cols
    w = splitmix64(seed, 2 * n)
    u1 = ((w[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = (w[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2) * sigma
    return z.astype(np.float16).view(np.uint16).reshape(rows, cols)


# The five workloads.  Sizes, code and exponent distributions, alpha, beta
# and C follow the statement of each case; `b_packed` marks the case that is
# run on the pre-shuffled B layout and `sa_packed` the one whose A scales are
# shuffled too (the operand set of the pages' pre-shuffled kernels).
WORKLOADS = {
    "tiny_128x256x512": dict(index=0, M=128, N=256, K=512, dist="uniform", e=(123, 131),
                             alpha=1.0, beta=0.0, c_sigma=None, b_packed=False, sa_packed=False),
    "mid_512x1024x2048": dict(index=1, M=512, N=1024, K=2048, dist="uniform", e=(123, 131),
                              alpha=1.0, beta=1.0, c_sigma=1.0, b_packed=False, sa_packed=False),
    "gemv_1x8192x8192": dict(index=2, M=1, N=8192, K=8192, dist="uniform", e=(120, 134),
                             alpha=0.5, beta=0.0, c_sigma=None, b_packed=False, sa_packed=False),
    "square_8192": dict(index=3, M=8192, N=8192, K=8192, dist="uniform", e=(123, 131),
                        alpha=1.0, beta=0.0, c_sigma=None, b_packed=True, sa_packed=True),
    "skinny_64x7168x16384": dict(index=4, M=64, N=7168, K=16384, dist="half_zero", e=(110, 140),
                                 alpha=1.0, beta=1.0, c_sigma=2.0, b_packed=False, sa_packed=False),
}


def make_problem(M: int, N: int, K: int, *, seed: int, dist: str = "uniform",
                 e=(123, 131), alpha: float = 1.0, beta: float = 0.0,
                 c_sigma: float | None = None, a_fmt: int = 0) -> dict:
    """Dense (unpadded) operands for one GEMM problem (A in format a_fmt:
    0 FP4, else see wide_codes; B is always FP4)."""
    lo, hi = e
    p = dict(M=M, N=N, K=K, alpha=float(alpha), beta=float(beta), seed=seed, a_fmt=a_fmt)
    if a_fmt == 0:
        p["A"] = fp4_codes_packed(_stream(seed, "A"), M, K, dist)
    else:
        p["A"] = wide_codes(_stream(seed, "A"), M, K, a_fmt)
    p["B"] = fp4_codes_packed(_stream(seed, "B"), N, K, dist)
    p["SA"] = e8m0_scales(_stream(seed, "SA"), M, K, lo, hi)
    p["SB"] = e8m0_scales(_stream(seed, "SB"), N, K, lo, hi)
    if c_sigma is not None:
        p["C"] = gaussian_bf16(_stream(seed, "C"), M, N, c_sigma)
    else:
        p["C"] = None
    return p


def make_workload(name: str) -> dict:
    w = WORKLOADS[name]
    p = make_problem(w["M"], w["N"], w["K"], seed=SEED_BASE + w["index"], dist=w["dist"],
                     e=w["e"], alpha=w["alpha"], beta=w["beta"], c_sigma=w["c_sigma"])
    p["name"] = name
    p["b_packed"] = w["b_packed"]
    p["sa_packed"] = w["sa_packed"]
    return p

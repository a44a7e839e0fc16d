"""Python access to the plain C oracle for the MXFP4 block-scaled GEMM.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU library never
imports, links or runs anything from this directory.

The arithmetic lives in ``mxfp4_oracle.c`` (plain fp64 triple loop, see its
header for the page passages it follows).  This module only marshals numpy
arrays and splits independent output columns across host threads (ctypes
releases the GIL while the C code runs), which changes no arithmetic: every
output element is computed by the same sequential k-ascending loop.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None
_lock = threading.Lock()


def build(force: bool = False) -> str:
    """Compile the oracle with the host C compiler (no GPU code involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["cc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB)
            i64, u8p, f64 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
            lib.oracle_e2m1.argtypes = [ctypes.c_uint]
            lib.oracle_e2m1.restype = f64
            lib.oracle_e8m0.argtypes = [ctypes.c_uint]
            lib.oracle_e8m0.restype = f64
            lib.oracle_bf16_rne.argtypes = [f64]
            lib.oracle_bf16_rne.restype = ctypes.c_uint16
            lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_bf16_to_double.restype = f64
            lib.oracle_fp4_code.argtypes = [u8p, i64, i64, i64]
            lib.oracle_fp4_code.restype = ctypes.c_uint
            lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_f16_to_double.restype = f64
            lib.oracle_f16_gemm.argtypes = [i64, u8p, i64, u8p, i64, u8p, i64, u8p, i64, u8p, u8p]
            lib.oracle_f16_gemm.restype = ctypes.c_int
            lib.oracle_decode.argtypes = [ctypes.c_int, ctypes.c_uint]
            lib.oracle_decode.restype = f64
            lib.oracle_format_bits.argtypes = [ctypes.c_int]
            lib.oracle_format_bits.restype = ctypes.c_int
            lib.oracle_elem_code.argtypes = [u8p, i64, ctypes.c_int, i64, i64]
            lib.oracle_elem_code.restype = ctypes.c_uint
            lib.oracle_mxgemm.argtypes = [i64, ctypes.c_int, u8p, i64, u8p, i64, u8p, i64, u8p, i64, ctypes.c_int,
                                          u8p, i64, ctypes.c_int, f64, f64, u8p, i64, u8p, i64,
                                          u8p, u8p, u8p]
            lib.oracle_mxgemm.restype = ctypes.c_int
            lib.oracle_dot_exact_parts.argtypes = [
                i64, u8p, i64, u8p, i64, u8p, i64, u8p, i64, i64, i64,
                ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_uint64),
                ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double),
                ctypes.POINTER(ctypes.c_uint16)]
            lib.oracle_dot_exact_parts.restype = ctypes.c_int
            lib.oracle_quantize_mxfp4.argtypes = [u8p, i64, i64, i64, u8p, i64, u8p, i64]
            lib.oracle_quantize_mxfp4.restype = None
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def e2m1(code: int) -> float:
    return _load().oracle_e2m1(code)


def e8m0(e: int) -> float:
    return _load().oracle_e8m0(e)


def bf16_rne(x: float) -> int:
    return int(_load().oracle_bf16_rne(float(x)))


def bf16_to_float(h: int) -> float:
    return _load().oracle_bf16_to_double(int(h) & 0xFFFF)


def fp4_code(X: np.ndarray, ld: int, r: int, k: int) -> int:
    X = np.ascontiguousarray(X, dtype=np.uint8)
    return int(_load().oracle_fp4_code(_ptr(X), ld, r, k))


# A formats (the library's ids): FP4 E2M1, FP8 E4M3, BF8 E5M2, FP6 E2M3, FP6 E3M2
FMT_FP4, FMT_E4M3, FMT_E5M2, FMT_E2M3, FMT_E3M2 = 0, 1, 2, 3, 4


def f16_to_float(h: int) -> float:
    return float(_load().oracle_f16_to_double(int(h)))


def f16_gemm(A, B, K, *, lda=None, ldb=None, rows=None, cols=None, threads=None):
    """Reference C = A B for fp16 bit patterns A [M, lda], B [K, ldb]
    (row-major, B K-major); returns (ref fp64, mag fp64) for rows x cols."""
    lib = _load()
    A = np.ascontiguousarray(A, dtype=np.uint16)
    B = np.ascontiguousarray(B, dtype=np.uint16)
    M, N = A.shape[0], B.shape[1]
    lda = A.shape[1] if lda is None else lda
    ldb = B.shape[1] if ldb is None else ldb
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.arange(N, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    nr, nc = len(rows), len(cols)
    ref = np.zeros((nr, nc), dtype=np.float64)
    mag = np.zeros((nr, nc), dtype=np.float64)
    if nr == 0 or nc == 0:
        return ref, mag
    threads = max(1, min(threads or min(16, os.cpu_count() or 1), nr))
    bounds = np.linspace(0, nr, threads + 1).astype(np.int64)

    def work(t):
        r0, r1 = int(bounds[t]), int(bounds[t + 1])
        if r1 <= r0:
            return
        rs = np.ascontiguousarray(rows[r0:r1])
        r_ = np.zeros((r1 - r0, nc), dtype=np.float64)
        m_ = np.zeros((r1 - r0, nc), dtype=np.float64)
        lib.oracle_f16_gemm(K, _ptr(A), lda, _ptr(B), ldb, _ptr(rs), r1 - r0, _ptr(cols), nc, _ptr(r_), _ptr(m_))
        ref[r0:r1], mag[r0:r1] = r_, m_

    ths = [threading.Thread(target=work, args=(t,)) for t in range(threads)]
    for th in ths:
        th.start()
    for th in ths:
        th.join()
    return ref, mag


def decode(fmt: int, code: int) -> float:
    return float(_load().oracle_decode(int(fmt), int(code)))


def format_bits(fmt: int) -> int:
    return int(_load().oracle_format_bits(int(fmt)))


def elem_code(X: np.ndarray, ld_bytes: int, bits: int, r: int, k: int) -> int:
    X = np.ascontiguousarray(X, dtype=np.uint8)
    return int(_load().oracle_elem_code(_ptr(X), int(ld_bytes), int(bits), int(r), int(k)))


def mxgemm(A, SA, B, SB, K, alpha=1.0, beta=0.0, C=None, *, lda=None, ldb=None,
           ldsa=None, ldsb=None, ldc=None, rows=None, cols=None, threads=None, a_fmt=FMT_FP4,
           b_layout=0):
    """Reference block of D for rows x cols.

    A: uint8 [M, lda * w / 8] for A's format (w = 4, 8 or 6 bits; lda counts
    elements), SA: uint8 [M, ldsa], B: uint8 [N, ldb/2] (FP4; with
    b_layout=1 MN-major: [K, ldb/2], row k holding the N columns' codes),
    SB: uint8 [N, ldsb], C: uint16 (bf16 bits) or float32 [M, ldc], or None.
    Returns (ref fp64, mag fp64, dref uint16) of shape [len(rows), len(cols)].
    """
    lib = _load()
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    SA = np.ascontiguousarray(SA, dtype=np.uint8)
    SB = np.ascontiguousarray(SB, dtype=np.uint8)
    M, N = A.shape[0], (B.shape[0] if b_layout == 0 else SB.shape[0])
    lda = A.shape[1] * 8 // format_bits(a_fmt) if lda is None else lda
    ldb = B.shape[1] * 2 if ldb is None else ldb
    ldsa = SA.shape[1] if ldsa is None else ldsa
    ldsb = SB.shape[1] if ldsb is None else ldsb
    c_f32 = 0
    if beta != 0.0:
        if C is None:
            raise ValueError("beta != 0 needs C")
        c_f32 = int(np.asarray(C).dtype == np.float32)
        C = np.ascontiguousarray(C, dtype=np.float32 if c_f32 else np.uint16)
        ldc = C.shape[1] if ldc is None else ldc
    else:
        ldc = 0 if ldc is None else ldc
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.arange(N, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    nr, nc = len(rows), len(cols)
    ref = np.zeros((nr, nc), dtype=np.float64)
    mag = np.zeros((nr, nc), dtype=np.float64)
    dref = np.zeros((nr, nc), dtype=np.uint16)
    if nr == 0 or nc == 0:
        return ref, mag, dref
    if threads is None:
        threads = max(1, min(16, os.cpu_count() or 1))
    threads = max(1, min(threads, nc))
    # Split the columns into contiguous slices; each thread fills its own
    # sub-arrays, which are copied into place afterwards.
    bounds = np.linspace(0, nc, threads + 1).astype(np.int64)
    outs = [None] * threads
    errs = []

    def work(t):
        c0, c1 = int(bounds[t]), int(bounds[t + 1])
        if c1 <= c0:
            outs[t] = None
            return
        cs = np.ascontiguousarray(cols[c0:c1])
        r_ = np.zeros((nr, c1 - c0), dtype=np.float64)
        m_ = np.zeros((nr, c1 - c0), dtype=np.float64)
        d_ = np.zeros((nr, c1 - c0), dtype=np.uint16)
        rc = lib.oracle_mxgemm(K, int(a_fmt), _ptr(A), lda, _ptr(SA), ldsa, _ptr(B), ldb, _ptr(SB), ldsb,
                               int(b_layout),
                               _ptr(C) if beta != 0.0 else None, ldc, c_f32, float(alpha), float(beta),
                               _ptr(rows), nr, _ptr(cs), c1 - c0,
                               _ptr(r_), _ptr(m_), _ptr(d_))
        if rc != 0:
            errs.append(rc)
        outs[t] = (c0, c1, r_, m_, d_)

    if threads == 1:
        work(0)
    else:
        ths = [threading.Thread(target=work, args=(t,)) for t in range(threads)]
        for th in ths:
            th.start()
        for th in ths:
            th.join()
    if errs:
        raise MemoryError("oracle could not allocate scratch memory")
    for o in outs:
        if o is None:
            continue
        c0, c1, r_, m_, d_ = o
        ref[:, c0:c1] = r_
        mag[:, c0:c1] = m_
        dref[:, c0:c1] = d_
    return ref, mag, dref


def dot_exact(A, SA, B, SB, K, i, j, *, lda=None, ldb=None, ldsa=None, ldsb=None):
    """Exact sum_k a(i,k) b(j,k) via 128-bit fixed point.

    Returns (mantissa:int, exp2:int, as_double:float, as_bf16:int) with
    sum = mantissa * 2**exp2 exactly, or raises ValueError (NaN scale or an
    exponent spread too wide for 128 bits)."""
    lib = _load()
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    SA = np.ascontiguousarray(SA, dtype=np.uint8)
    SB = np.ascontiguousarray(SB, dtype=np.uint8)
    lda = A.shape[1] * 2 if lda is None else lda
    ldb = B.shape[1] * 2 if ldb is None else ldb
    ldsa = SA.shape[1] if ldsa is None else ldsa
    ldsb = SB.shape[1] if ldsb is None else ldsb
    hi, lo, e = ctypes.c_int64(), ctypes.c_uint64(), ctypes.c_int()
    d, h = ctypes.c_double(), ctypes.c_uint16()
    rc = lib.oracle_dot_exact_parts(K, _ptr(A), lda, _ptr(SA), ldsa, _ptr(B), ldb, _ptr(SB), ldsb,
                                    int(i), int(j), ctypes.byref(hi), ctypes.byref(lo),
                                    ctypes.byref(e), ctypes.byref(d), ctypes.byref(h))
    if rc:
        raise ValueError("exact mode unavailable (code %d)" % rc)
    mant = (hi.value << 64) | lo.value
    return mant, e.value, d.value, int(h.value)


def quantize_mxfp4(X, K=None, *, ldx=None):
    """bf16 [M, ldx] (uint16 bit patterns) -> (A [M, K/2] uint8 fp4x2,
    S [M, K/32] uint8 E8M0), by the conversion rule in mxfp4_oracle.c
    (readings Q1-Q4 there)."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    M = X.shape[0]
    ldx = X.shape[1] if ldx is None else ldx
    K = ldx if K is None else K
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    A = np.zeros((M, K // 2), dtype=np.uint8)
    S = np.zeros((M, K // 32), dtype=np.uint8)
    _load().oracle_quantize_mxfp4(_ptr(X), M, K, ldx, _ptr(A), K, _ptr(S), K // 32)
    return A, S

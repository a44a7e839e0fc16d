"""Python binding of libmxgemm (MXFP4 block-scaled GEMM for gfx950).

Argument marshalling only: every function below calls the C-ABI entry point
of the same name in libmxgemm.so (declared in include/libmxgemm.h) and every
step of the computation runs in the library's HIP kernels.  Tensors may be
passed as torch tensors (their data_ptr() is used) or as raw device
addresses (int).  The stream defaults to torch's current stream.

There is no fallback: if libmxgemm.so is missing or fails to load, every
call raises MxGemmError.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxgemm.so")

# C-ABI entry points declared in include/libmxgemm.h
EXPORTS = ("mxgemm_status_string", "mxgemm_run", "mxgemm_run_noalloc", "mxgemm_run_bf16a", "mxgemm_pack_b", "mxgemm_pack_scales", "mxgemm_pack_a",
           "mxgemm_pack_a_bytes", "mxgemm_quantize",
           "mxgemm_f16_run", "mxgemm_query", "mxgemm_plan", "mxgemm_query_ex", "mxgemm_plan_ex",
           "mxgemm_stream_read", "mxgemm_release_workspaces")

STATUS = {0: "MXGEMM_OK", -1: "MXGEMM_ERR_INVALID_ARG", -2: "MXGEMM_ERR_SHAPE",
          -3: "MXGEMM_ERR_ALIGN", -4: "MXGEMM_ERR_UNSUPPORTED_DEVICE", -5: "MXGEMM_ERR_HIP",
          -6: "MXGEMM_ERR_WORKSPACE", -7: "MXGEMM_ERR_SCRATCH"}


class MxGemmError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = status
        name = STATUS.get(status, str(status))
        super().__init__("%s failed: %s (%s)" % (where, name, _status_text(status)))


class Strides(ctypes.Structure):
    _fields_ = [("ldd", ctypes.c_int64), ("ldc", ctypes.c_int64), ("lda", ctypes.c_int64),
                ("ldb", ctypes.c_int64), ("ldsa", ctypes.c_int64), ("ldsb", ctypes.c_int64),
                ("b_packed", ctypes.c_int32), ("sa_packed", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("c_f32", ctypes.c_int32), ("split_mode", ctypes.c_int32),
                ("a_format", ctypes.c_int32), ("b_layout", ctypes.c_int32), ("a_packed", ctypes.c_int32)]


SPLIT_FP32 = 0         # MXGEMM_SPLIT_FP32
SPLIT_BF16_ATOMIC = 1  # MXGEMM_SPLIT_BF16_ATOMIC
# MXGEMM_FMT_*: A's element format
FMT_FP4, FMT_FP8_E4M3, FMT_FP8_E5M2, FMT_FP6_E2M3, FMT_FP6_E3M2 = 0, 1, 2, 3, 4
FORMAT_BITS = (4, 8, 8, 6, 6)
B_NK, B_KN = 0, 1  # MXGEMM_B_NK, MXGEMM_B_KN
NOALLOC_SCRATCH_BYTES = 32 << 20  # MXGEMM_NOALLOC_SCRATCH_BYTES


class Info(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t), ("packed_b_bytes", ctypes.c_size_t),
                ("packed_sb_bytes", ctypes.c_size_t), ("packed_sa_bytes", ctypes.c_size_t),
                ("num_cu", ctypes.c_int32),
                ("persist_grid", ctypes.c_int32), ("kernel_name", ctypes.c_char * 64),
                ("arch", ctypes.c_char * 32), ("peak_flops", ctypes.c_double),
                ("clock_hz", ctypes.c_double)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["kernel_name"] = self.kernel_name.decode()
        d["arch"] = self.arch.decode()
        return d


_lib = None


def lib():
    """The loaded libmxgemm.so (raises MxGemmError if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MxGemmError(-5, "loading %s (not built; run __graft_entry__.build())" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.mxgemm_status_string.argtypes = [i32]
        L.mxgemm_status_string.restype = ctypes.c_char_p
        L.mxgemm_run.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, i32, i32, i32,
                                 ctypes.POINTER(Strides), i32, vp]
        L.mxgemm_run.restype = i32
        L.mxgemm_run_noalloc.argtypes = L.mxgemm_run.argtypes
        L.mxgemm_run_noalloc.restype = i32
        L.mxgemm_run_bf16a.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, i32, i32, i32, i64,
                                       ctypes.POINTER(Strides), i32, vp]
        L.mxgemm_run_bf16a.restype = i32
        L.mxgemm_pack_b.argtypes = [vp, vp, vp, vp, i32, i32, i64, i64, vp]
        L.mxgemm_pack_b.restype = i32
        L.mxgemm_pack_scales.argtypes = [vp, vp, i32, i32, i64, vp]
        L.mxgemm_pack_scales.restype = i32
        L.mxgemm_pack_a.argtypes = [vp, vp, vp, vp, i32, i32, i64, i64, i32, vp]
        L.mxgemm_pack_a.restype = i32
        L.mxgemm_pack_a_bytes.argtypes = [i32, i32]
        L.mxgemm_pack_a_bytes.restype = ctypes.c_size_t
        L.mxgemm_quantize.argtypes = [vp, vp, vp, i32, i32, i64, i64, i64, vp]
        L.mxgemm_quantize.restype = i32
        L.mxgemm_f16_run.argtypes = [vp, vp, vp, i32, i32, i32, i64, i64, i64, vp]
        L.mxgemm_f16_run.restype = i32
        L.mxgemm_query.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(Info)]
        L.mxgemm_query.restype = i32
        L.mxgemm_plan.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(Info)]
        L.mxgemm_plan.restype = i32
        L.mxgemm_query_ex.argtypes = [i32, i32, i32, ctypes.POINTER(Strides), i32, ctypes.POINTER(Info)]
        L.mxgemm_query_ex.restype = i32
        L.mxgemm_plan_ex.argtypes = [i32, i32, i32, ctypes.POINTER(Strides), i32, i32, ctypes.POINTER(Info)]
        L.mxgemm_plan_ex.restype = i32
        L.mxgemm_stream_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        L.mxgemm_stream_read.restype = i32
        L.mxgemm_release_workspaces.argtypes = []
        L.mxgemm_release_workspaces.restype = i32
        _lib = L
    return _lib


def _status_text(status):
    try:
        return lib().mxgemm_status_string(status).decode()
    except Exception:
        return "?"


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where):
    if status != 0:
        raise MxGemmError(status, where)


def make_strides(*, ldd, ldc, lda, ldb, ldsa, ldsb, b_packed=0, sa_packed=0, workspace=None,
                 workspace_bytes=0, c_f32=0, split_mode=SPLIT_FP32, a_format=FMT_FP4, b_layout=B_NK, a_packed=0):
    return Strides(ldd, ldc, lda, ldb, ldsa, ldsb, b_packed, sa_packed, _ptr(workspace), workspace_bytes,
                   c_f32, split_mode, a_format, b_layout, a_packed)


def mxgemm_status_string(status: int) -> str:
    return lib().mxgemm_status_string(status).decode()


def mxgemm_run(D, C, A, B, scaleA, scaleB, alpha, beta, M, N, K, strides=None, split_k=-1,
               stream=None, check=True):
    """D = bf16(alpha * A * B^T + beta * C) on `stream` (asynchronous)."""
    sp = ctypes.byref(strides) if strides is not None else None
    st = lib().mxgemm_run(_ptr(D), _ptr(C), _ptr(A), _ptr(B), _ptr(scaleA), _ptr(scaleB),
                          float(alpha), float(beta), int(M), int(N), int(K), sp, int(split_k),
                          _stream(stream))
    if check:
        _check(st, "mxgemm_run")
    return st


def mxgemm_run_noalloc(D, C, A, B, scaleA, scaleB, alpha, beta, M, N, K, strides=None, split_k=-1,
                       stream=None, check=True):
    """mxgemm_run with the library's buffers in its fixed device scratch (no allocation)."""
    sp = ctypes.byref(strides) if strides is not None else None
    st = lib().mxgemm_run_noalloc(_ptr(D), _ptr(C), _ptr(A), _ptr(B), _ptr(scaleA), _ptr(scaleB),
                                  float(alpha), float(beta), int(M), int(N), int(K), sp, int(split_k),
                                  _stream(stream))
    if check:
        _check(st, "mxgemm_run_noalloc")
    return st


def mxgemm_pack_b(Bp, SBp, B, scaleB, N, K, ldb=None, ldsb=None, stream=None, check=True):
    """Pre-shuffle B and its scales into the kernels' layout (asynchronous)."""
    ldb = K if ldb is None else ldb
    ldsb = K // 32 if ldsb is None else ldsb
    st = lib().mxgemm_pack_b(_ptr(Bp), _ptr(SBp), _ptr(B), _ptr(scaleB), int(N), int(K),
                             int(ldb), int(ldsb), _stream(stream))
    if check:
        _check(st, "mxgemm_pack_b")
    return st


def mxgemm_pack_scales(Sp, S, rows, K, lds=None, stream=None, check=True):
    """Shuffle a [rows][K/32] scale matrix into the packed scale layout
    (scaleA for sa_packed = 1; asynchronous)."""
    lds = K // 32 if lds is None else lds
    st = lib().mxgemm_pack_scales(_ptr(Sp), _ptr(S), int(rows), int(K), int(lds), _stream(stream))
    if check:
        _check(st, "mxgemm_pack_scales")
    return st


def mxgemm_pack_a(Ap, SAp, A, scaleA, M, K, a_format, lda=None, ldsa=None, stream=None, check=True):
    """Put an FP6 A and its scales into the dense FP6 tile's order, for
    mxgemm_run with a_packed = 1 (asynchronous)."""
    lda = K if lda is None else lda
    ldsa = K // 32 if ldsa is None else ldsa
    st = lib().mxgemm_pack_a(_ptr(Ap), _ptr(SAp), _ptr(A), _ptr(scaleA), int(M), int(K), int(lda), int(ldsa),
                             int(a_format), _stream(stream))
    if check:
        _check(st, "mxgemm_pack_a")
    return st


def mxgemm_pack_a_bytes(M, K) -> int:
    return int(lib().mxgemm_pack_a_bytes(int(M), int(K)))


def mxgemm_run_bf16a(D, C, X, B, scaleB, alpha, beta, M, N, K, ldx=None, strides=None, split_k=-1,
                     stream=None, check=True):
    """D = bf16(alpha * quantize(X) * B^T + beta * C) on `stream` (asynchronous);
    X is a bf16 [M, ldx] activation (one fused launch at M = 1)."""
    sp = ctypes.byref(strides) if strides is not None else None
    st = lib().mxgemm_run_bf16a(_ptr(D), _ptr(C), _ptr(X), _ptr(B), _ptr(scaleB), float(alpha), float(beta),
                                int(M), int(N), int(K), int(K if ldx is None else ldx), sp, int(split_k),
                                _stream(stream))
    if check:
        _check(st, "mxgemm_run_bf16a")
    return st


def mxgemm_quantize(A, SA, X, M, K, ldx=None, lda=None, ldsa=None, stream=None, check=True):
    """bf16 X [M][ldx] -> packed E2M1 A [M][lda/2] bytes and E8M0 scales
    SA [M][ldsa] (asynchronous; strides default to dense rows)."""
    ldx = K if ldx is None else ldx
    lda = K if lda is None else lda
    ldsa = K // 32 if ldsa is None else ldsa
    st = lib().mxgemm_quantize(_ptr(A), _ptr(SA), _ptr(X), int(M), int(K), int(ldx), int(lda),
                               int(ldsa), _stream(stream))
    if check:
        _check(st, "mxgemm_quantize")
    return st


def mxgemm_f16_run(C, A, B, M, N, K, lda=None, ldb=None, ldc=None, stream=None, check=True):
    """fp32 C [M][ldc] = fp16 A [M][lda] x fp16 B [K][ldb] (asynchronous;
    strides in elements, default dense)."""
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    st = lib().mxgemm_f16_run(_ptr(C), _ptr(A), _ptr(B), int(M), int(N), int(K), int(lda), int(ldb), int(ldc),
                              _stream(stream))
    if check:
        _check(st, "mxgemm_f16_run")
    return st


def mxgemm_query(M, N, K, b_packed=0, split_k=-1) -> dict:
    info = Info()
    _check(lib().mxgemm_query(int(M), int(N), int(K), int(b_packed), int(split_k),
                              ctypes.byref(info)), "mxgemm_query")
    return info.as_dict()


def mxgemm_query_ex(M, N, K, strides=None, split_k=-1) -> dict:
    """mxgemm_query for the path mxgemm_run takes with these strides/options."""
    info = Info()
    sp = ctypes.byref(strides) if strides is not None else None
    _check(lib().mxgemm_query_ex(int(M), int(N), int(K), sp, int(split_k), ctypes.byref(info)), "mxgemm_query_ex")
    return info.as_dict()


def mxgemm_plan_ex(M, N, K, strides=None, split_k=-1, num_cu=256) -> dict:
    """mxgemm_plan for the path mxgemm_run takes with these strides/options."""
    info = Info()
    sp = ctypes.byref(strides) if strides is not None else None
    _check(lib().mxgemm_plan_ex(int(M), int(N), int(K), sp, int(split_k), int(num_cu), ctypes.byref(info)),
           "mxgemm_plan_ex")
    return info.as_dict()


def mxgemm_plan(M, N, K, b_packed=0, split_k=-1, num_cu=256) -> dict:
    info = Info()
    _check(lib().mxgemm_plan(int(M), int(N), int(K), int(b_packed), int(split_k), int(num_cu),
                             ctypes.byref(info)), "mxgemm_plan")
    return info.as_dict()


def mxgemm_stream_read(src, nbytes, sink, stream=None, check=True):
    """Streaming read of nbytes at src (the achievable-bandwidth reference)."""
    st = lib().mxgemm_stream_read(_ptr(src), int(nbytes), _ptr(sink), _stream(stream))
    if check:
        _check(st, "mxgemm_stream_read")
    return st


def mxgemm_release_workspaces():
    _check(lib().mxgemm_release_workspaces(), "mxgemm_release_workspaces")

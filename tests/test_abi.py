"""Host-side checks of the C-ABI library (no GPU needed, no compute calls).

- libmxgemm.so loads and exports every function include/libmxgemm.h declares;
- every argument error is reported before any HIP call is made;
- the planner (mxgemm_plan, pure host logic) makes choices that respect its
  contract on the five workloads and on edge shapes.
"""
import ctypes
import os
import re

import pytest

import block_scaled_precision_mxfp4_amd as mx
from block_scaled_precision_mxfp4_amd import build as mxbuild
from block_scaled_precision_mxfp4_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmxgemm.h")


@pytest.fixture(scope="module", autouse=True)
def built():
    if mxbuild.is_stale():
        mxbuild.build()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxgemm_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(mx.EXPORTS) == declared_functions()


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mx.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        s = mx.mxgemm_status_string(code)
        assert s and s != "unknown status"
    assert mx.mxgemm_status_string(-99) == "unknown status"


def _run(**kw):
    args = dict(D=0x1000, C=None, A=0x2000, B=0x3000, scaleA=0x4000, scaleB=0x5000,
                alpha=1.0, beta=0.0, M=128, N=256, K=512, strides=None, split_k=-1, stream=0)
    args.update(kw)
    return mx.mxgemm_run(**args, check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(D=None), -1), (dict(A=None), -1), (dict(B=None), -1), (dict(scaleA=None), -1),
    (dict(scaleB=None), -1), (dict(beta=1.0, C=None), -1), (dict(split_k=3), -1),
    (dict(split_k=32), -1), (dict(split_k=-2), -1),
    (dict(M=0), -2), (dict(N=0), -2), (dict(K=0), -2), (dict(K=16), -2), (dict(K=48), -2),
    (dict(K=(1 << 24) + 32), -2),
    (dict(A=0x2008), -3), (dict(B=0x3004), -3), (dict(D=0x1001), -3),
])
def test_run_validation_before_any_hip_call(kw, code):
    assert _run(**kw) == code


def test_run_stride_validation():
    def st(**kw):
        d = dict(ldd=256, ldc=256, lda=512, ldb=512, ldsa=16, ldsb=16)
        d.update(kw)
        return mx.make_strides(**d)
    assert _run(strides=st(ldd=255)) == -2
    assert _run(strides=st(lda=480)) == -2
    assert _run(strides=st(ldsa=15)) == -2
    assert _run(strides=st(ldb=510)) == -2
    assert _run(strides=st(ldsb=15)) == -2
    assert _run(strides=st(ldc=255), beta=1.0, C=0x6000) == -2
    assert _run(strides=st(lda=513)) == -3      # odd element stride
    assert _run(strides=st(lda=528)) == -3      # 264-byte pitch: not a multiple of 16
    assert _run(strides=st(ldb=528)) == -3
    s = st()
    s.sa_packed = 2
    assert _run(strides=s) == -1
    s = st()
    s.sa_packed = 1  # packed A scales come with packed B only
    assert _run(strides=s) == -1
    # packed A scales: ldsa is ignored, scaleA must be 4-byte aligned
    assert _run(strides=st(ldsa=0, ldb=0, ldsb=0, b_packed=1, sa_packed=1), scaleA=0x4002) == -3
    s = st()
    s.b_packed = 2
    assert _run(strides=s) == -1
    # packed B: B strides are ignored, but scaleB must be 4-byte aligned
    assert _run(strides=st(ldb=0, ldsb=0, b_packed=1), scaleB=0x5002) == -3
    # option fields: 0 or 1 only
    assert _run(strides=st(c_f32=2)) == -1
    assert _run(strides=st(split_mode=2)) == -1
    assert _run(strides=st(split_mode=-1)) == -1
    # an f32 C needs 4-byte alignment (a bf16 C: 2)
    assert _run(strides=st(c_f32=1), beta=1.0, C=0x6002) == -3
    # A formats: 0..4; wider formats need row-major A scales and the fp32 split;
    # b_layout is 0 or 1 (MN-major B needs FP4 A); A's byte pitch lda * w / 8 a multiple of 16
    assert _run(strides=st(a_format=5)) == -1
    assert _run(strides=st(a_format=-1)) == -1
    s = st(a_format=1)
    s.b_layout = 2
    assert _run(strides=s) == -1
    assert _run(strides=st(b_layout=1, a_format=1)) == -1
    # MN-major B: ldb counts the N columns of a K-row (>= N, even, a 16-byte pitch)
    assert _run(strides=st(b_layout=1, ldb=255)) == -2
    assert _run(strides=st(b_layout=1, ldb=264)) == -3      # 132-byte pitch
    assert _run(strides=st(b_layout=1, ldb=256)) not in (-1, -2, -3)
    assert _run(strides=st(b_layout=1, ldb=1 << 24), K=512) == -2  # 256 K-rows reach 2^31 bytes
    assert _run(strides=st(a_format=1, ldsa=0, ldb=0, ldsb=0, b_packed=1, sa_packed=1)) == -1
    assert _run(strides=st(a_format=2, split_mode=1)) == -1
    assert _run(strides=st(a_format=1, lda=520)) == -3   # 520-byte pitch
    assert _run(strides=st(a_format=3, lda=516)) == -3   # 387-byte pitch
    assert _run(strides=st(a_format=4, lda=528)) == -3   # 396 bytes: not a multiple of 8
    assert _run(strides=st(a_format=4, lda=510)) == -2   # lda < K
    # every byte range of a 256-row tile stays below 2^31: scale row pitches
    assert _run(strides=st(ldsa=1 << 23)) == -2
    assert _run(strides=st(ldsb=1 << 23)) == -2
    # (just below the limit validation passes; the call then fails for want
    # of a device here)
    assert _run(strides=st(ldsa=(1 << 23) - 1, ldsb=(1 << 23) - 1)) not in (-1, -2, -3)
    # bf16-atomic split-K: D 4-byte aligned, ldd and N even
    assert _run(strides=st(split_mode=1), D=0x1002) == -3
    assert _run(strides=st(split_mode=1, ldd=257)) == -3
    assert _run(strides=st(split_mode=1), N=255) == -3


def test_struct_layouts_match_the_header():
    """The binding's ctypes structs have the C header's size and field
    offsets (compiled with the host C compiler)."""
    import shutil
    import subprocess
    import tempfile
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    fields = {"mxgemm_strides": mx.Strides, "mxgemm_info": mx.Info}
    lines = []
    for cname, cls in fields.items():
        lines.append('printf("%%zu\\n", sizeof(%s));' % cname)
        for f, _ in cls._fields_:
            lines.append('printf("%%zu\\n", offsetof(%s, %s));' % (cname, f))
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"libmxgemm.h\"\nint main(void){%s return 0;}\n" % " ".join(lines)
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "l.c"), os.path.join(d, "l")
        open(c, "w").write(src)
        r = subprocess.run([cc, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.dirname(HEADER),
                            c, "-o", exe], capture_output=True, text=True)
        if r.returncode != 0:
            pytest.skip("header does not compile here: " + r.stderr[:200])
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    want = []
    for cname, cls in fields.items():
        want.append(ctypes.sizeof(cls))
        want += [getattr(cls, f).offset for f, _ in cls._fields_]
    assert got == want


def test_pack_validation_before_any_hip_call():
    f = lambda **kw: mx.mxgemm_pack_b(**dict(dict(Bp=0x1000, SBp=0x2000, B=0x3000, scaleB=0x4000,
                                                   N=64, K=256, stream=0), **kw), check=False)
    assert f(Bp=None) == -1 and f(SBp=None) == -1 and f(B=None) == -1 and f(scaleB=None) == -1
    assert f(N=0) == -2 and f(K=40) == -2 and f(ldb=128) == -2 and f(ldsb=4) == -2
    assert f(Bp=0x1008) == -3 and f(SBp=0x2002) == -3 and f(B=0x3008) == -3 and f(ldb=272) == -3


def test_pack_scales_validation_before_any_hip_call():
    f = lambda **kw: mx.mxgemm_pack_scales(**dict(dict(Sp=0x1000, S=0x2000, rows=64, K=256, stream=0), **kw),
                                           check=False)
    assert f(Sp=None) == -1 and f(S=None) == -1
    assert f(rows=0) == -2 and f(K=40) == -2 and f(lds=4) == -2
    assert f(Sp=0x1002) == -3


def test_f16_validation_before_any_hip_call():
    f = lambda **kw: mx.mxgemm_f16_run(**dict(dict(C=0x1000, A=0x2000, B=0x3000, M=64, N=64, K=64,
                                                   lda=None, ldb=None, ldc=None, stream=0), **kw), check=False)
    assert f(C=None) == -1 and f(A=None) == -1 and f(B=None) == -1
    assert f(M=0) == -2 and f(K=60) == -2 and f(N=60) == -2 and f(lda=32) == -2 and f(ldc=60) == -2
    assert f(A=0x2008) == -3 and f(C=0x1002) == -3 and f(lda=72 + 4) == -3 and f(ldb=68) == -3


def test_quantize_validation_before_any_hip_call():
    f = lambda **kw: mx.mxgemm_quantize(**dict(dict(A=0x1000, SA=0x2000, X=0x3000, M=64, K=256, stream=0),
                                              **kw), check=False)
    assert f(A=None) == -1 and f(SA=None) == -1 and f(X=None) == -1
    assert f(M=0) == -2 and f(K=40) == -2 and f(K=0) == -2 and f(ldx=128) == -2 and f(lda=128) == -2
    assert f(ldsa=4) == -2
    # X rows in whole 16-byte chunks, A as mxgemm_run requires it
    assert f(X=0x3008) == -3 and f(ldx=260) == -3 and f(A=0x1008) == -3 and f(lda=257) == -3
    assert f(lda=272) == -3
    assert f(SA=0x2001, ldsa=9) != -3  # scales need no alignment (no device here: -4 or -5)


def test_query_and_plan_argument_errors():
    info = mx.Info()
    L = mx.lib()
    assert L.mxgemm_plan(8, 8, 64, 0, -1, 256, None) == -1
    assert L.mxgemm_plan(8, 8, 64, 2, -1, 256, ctypes.byref(info)) == -1
    assert L.mxgemm_plan(8, 8, 64, 0, 5, 256, ctypes.byref(info)) == -1
    assert L.mxgemm_plan(8, 8, 64, 0, -1, 0, ctypes.byref(info)) == -1
    assert L.mxgemm_plan(8, 8, 40, 0, -1, 256, ctypes.byref(info)) == -2
    assert L.mxgemm_query(0, 8, 64, 0, -1, ctypes.byref(info)) == -2


def cdiv(a, b):
    return -(-a // b)


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_plan_for_workloads(name):
    w = inputs.WORKLOADS[name]
    M, N, K = w["M"], w["N"], w["K"]
    for b_packed in (0, 1):
        p = mx.mxgemm_plan(M, N, K, b_packed, -1, 256)
        assert p["split_k"] in (1, 2, 4, 8, 16)
        if M == 1 and not b_packed and K % 2048 == 0 and cdiv(N, 4) >= 256:
            # the single-row GEMV: 4 rows of B per workgroup, unsplit
            assert p["kernel"] == 4 and p["kernel_name"] == "gemv_m1_n4"
            assert (p["tile_m"], p["tile_n"], p["split_k"]) == (1, 4, 1)
        elif M <= 16:
            assert p["kernel"] == 1 and p["kernel_name"].startswith("skinny")
            assert p["tile_m"] >= M
        elif M <= 64:
            assert p["kernel"] == 2 and p["kernel_name"].startswith("rows")
            assert p["tile_m"] >= M and p["tile_n"] in (64, 128)
        else:
            assert p["kernel"] == 0 and p["kernel_name"].startswith("tile")
        tiles = cdiv(M, p["tile_m"]) * cdiv(N, p["tile_n"]) if M > 64 else cdiv(N, p["tile_n"])
        assert p["grid"] == tiles * p["split_k"]
        if p["split_k"] > 1:
            part = p["tile_m"] * p["tile_n"] * 4 if M > 64 else p["tile_n"] * cdiv(M, 16) * 16 * 4
            assert p["workspace_bytes"] == tiles * p["split_k"] * part
        else:
            assert p["workspace_bytes"] == 0
        assert p["packed_b_bytes"] == cdiv(N, 16) * 16 * cdiv(K // 32, 4) * 64
        assert p["packed_sb_bytes"] == cdiv(N, 32) * 32 * cdiv(K // 32, 8) * 8
    # the large square case fills the machine with full tiles and no split
    if name == "square_8192":
        p = mx.mxgemm_plan(M, N, K, 1, -1, 256)
        assert (p["tile_m"], p["tile_n"], p["split_k"]) == (256, 256, 1)
    # the skinny cases get enough workgroups to cover most CUs
    if M <= 64:
        assert mx.mxgemm_plan(M, N, K, 0, -1, 256)["grid"] * 5 >= 4 * 256


@pytest.mark.parametrize("s", [1, 2, 4, 8, 16])
def test_forced_split_is_honoured_or_reduced(s):
    # K = 4096: 128 blocks; the tiled kernel splits in 8-block units (up to
    # 16 chunks), the skinny one in 16-block units (up to 8 chunks)
    assert mx.mxgemm_plan(300, 500, 4096, 0, s, 256)["split_k"] == s
    assert mx.mxgemm_plan(1, 500, 4096, 0, s, 256)["split_k"] == min(s, 8)
    assert mx.mxgemm_plan(1, 500, 8192, 0, s, 256)["split_k"] == s
    # K = 256: a single 256-K stage; any split collapses to 1
    assert mx.mxgemm_plan(300, 500, 256, 0, s, 256)["split_k"] == 1
    # K = 1024: 32 blocks -> at most 4 chunks of 8
    assert mx.mxgemm_plan(300, 500, 1024, 0, s, 256)["split_k"] == min(s, 4)


def test_plan_is_deterministic():
    a = [mx.mxgemm_plan(m, n, k, 0, -1, 256) for m, n, k in [(77, 999, 2048), (4096, 4096, 4096)]]
    b = [mx.mxgemm_plan(m, n, k, 0, -1, 256) for m, n, k in [(77, 999, 2048), (4096, 4096, 4096)]]
    assert a == b


def test_persistent_form_is_planned_only_where_it_applies(monkeypatch):
    """The 256 x 256 tiled kernel's persistent form: whole unsplit tiles,
    an even number of 8-block stages, more tiles than CUs, and a staged
    epilogue (ldd % 8 == 0)."""
    st = lambda N, K, ldd=None, pk=1: mx.make_strides(ldd=ldd or N, ldc=N, lda=K, ldb=K, ldsa=K // 32,
                                                       ldsb=K // 32, b_packed=pk, sa_packed=pk)
    pg = lambda M, N, K, s, split=-1: mx.mxgemm_plan_ex(M, N, K, s, split, 256)["persist_grid"]
    assert pg(8192, 8192, 8192, st(8192, 8192)) == 256
    assert mx.mxgemm_plan(8192, 8192, 8192, 1, -1, 256)["persist_grid"] == 0    # row-major A scales
    assert pg(5120, 5120, 512, st(5120, 512, pk=0)) == 0            # 256 x 256 needs packed B and A scales
    assert pg(5120, 5120, 512, st(5120, 512)) == 256
    monkeypatch.setenv("MXGEMM_FORCE_TILE", "1")
    assert pg(4352, 4352, 1024, st(4352, 1024)) == 0                # 256 x 128 tile: plain grid
    monkeypatch.delenv("MXGEMM_FORCE_TILE")
    assert pg(4352, 4352, 1024, st(4352, 1024)) == 256
    assert pg(8192, 8192, 8192, st(8192, 8192), split=2) == 0      # split K
    assert pg(8192, 8192, 8448, st(8192, 8448)) == 0               # 264 blocks: odd stage count
    assert pg(8192, 8200, 8192, st(8200, 8192)) == 0               # ragged N tile
    assert pg(4096, 4096, 4096, st(4096, 4096)) == 0               # one round of tiles
    assert pg(8192, 8192, 8192, st(8192, 8192, ldd=8196)) == 0     # unstaged epilogue
    assert mx.mxgemm_plan_ex(8192, 8192, 8192, st(8192, 8192), -1, 128)["persist_grid"] == 128
    # MN-major B codes with packed scales: persistent too; with row-major scales not
    kn = lambda pk: mx.make_strides(ldd=8192, ldc=8192, lda=8192, ldb=8192, ldsa=256, ldsb=256, b_packed=pk,
                                    sa_packed=pk, b_layout=mx.B_KN)
    assert pg(8192, 8192, 8192, kn(1)) == 256
    assert pg(8192, 8192, 8192, kn(0)) == 0
    monkeypatch.setenv("MXGEMM_TILE_PERSIST", "0")
    assert pg(8192, 8192, 8192, st(8192, 8192)) == 0


def test_run_bf16a_validation_before_any_hip_call():
    def f(**kw):
        args = dict(D=0x1000, C=None, X=0x2000, B=0x3000, scaleB=0x5000, alpha=1.0, beta=0.0, M=1, N=256,
                    K=512, ldx=None, strides=None, split_k=-1, stream=0)
        args.update(kw)
        return mx.mxgemm_run_bf16a(**args, check=False)
    st = lambda **kw: mx.make_strides(**dict(dict(ldd=256, ldc=256, lda=512, ldb=512, ldsa=16, ldsb=16), **kw))
    assert f(X=None) == -1 and f(B=None) == -1 and f(scaleB=None) == -1 and f(D=None) == -1
    assert f(beta=1.0) == -1 and f(split_k=3) == -1
    for M in (1, 8):
        # A's options must stay at their defaults: the row is quantized to FP4 with row-major scales
        assert f(M=M, strides=st(a_format=mx.FMT_FP8_E4M3)) == -1
        assert f(M=M, strides=st(b_packed=1, sa_packed=1)) == -1
        assert f(M=M, K=48) == -2 and f(M=M, N=0) == -2
    assert f(strides=st(split_mode=mx.SPLIT_BF16_ATOMIC)) == -1
    assert f(ldx=480) == -2                      # ldx < K
    assert f(X=0x2008) == -3 and f(ldx=516) == -3  # 16-byte rows of X


def test_stream_read_validation_before_any_hip_call():
    f = lambda **kw: mx.mxgemm_stream_read(**dict(dict(src=0x1000, nbytes=4096, sink=0x2000, stream=0), **kw),
                                           check=False)
    assert f(src=None) == -1 and f(sink=None) == -1
    assert f(nbytes=0) == -2 and f(nbytes=4100) == -2 and f(nbytes=1 << 31) == -2
    assert f(src=0x1008) == -3 and f(sink=0x2002) == -3
    assert f() not in (-1, -2, -3)


def test_prepacked_fp6_A_plan_and_sizes():
    """a_packed = 1 (an FP6 A from mxgemm_pack_a): planned on the dense FP6
    tile whatever the cost model would pick, refused for FP4/FP8 A and for
    M <= 64; mxgemm_pack_a_bytes = ceil(M/16) x even 128-K steps x 1536."""
    def st(fmt, a_packed):
        return mx.make_strides(ldd=2048, ldc=2048, lda=4096, ldb=4096, ldsa=128, ldsb=128, b_packed=1,
                               a_format=fmt, a_packed=a_packed)
    # the cost model keeps 2048 x 2048 x 4096 FP6 on the 128 x 128 tile
    assert mx.mxgemm_plan_ex(2048, 2048, 4096, st(mx.FMT_FP6_E2M3, 0))["kernel_name"] != "tile_fp6_256x256"
    for fmt in (mx.FMT_FP6_E2M3, mx.FMT_FP6_E3M2):
        assert mx.mxgemm_plan_ex(2048, 2048, 4096, st(fmt, 1))["kernel_name"] == "tile_fp6_256x256"
    for fmt, M in ((mx.FMT_FP4, 2048), (mx.FMT_FP8_E4M3, 2048), (mx.FMT_FP6_E2M3, 64), (mx.FMT_FP6_E2M3, 1)):
        with pytest.raises(mx.MxGemmError):
            mx.mxgemm_plan_ex(M, 2048, 4096, st(fmt, 1))
    with pytest.raises(mx.MxGemmError):
        mx.mxgemm_plan_ex(2048, 2048, 4096, st(mx.FMT_FP6_E2M3, 2))
    assert mx.mxgemm_pack_a_bytes(33, 1056) == 3 * 10 * 1536  # 33 blocks -> 5 8-block stages -> 10 steps
    assert mx.mxgemm_pack_a_bytes(8192, 8192) == 512 * 64 * 1536
    assert mx.mxgemm_pack_a_bytes(0, 1024) == 0


def test_gemv_plan_conditions_host():
    """The GEMV's planner conditions on the host (256 CUs): M == 1 (any A
    format) or 2 <= M <= 8 (FP4 A), row-major B, K % 2048 == 0, unsplit or
    split 1, N >= 4 x CUs."""
    name = lambda M, N, K, packed=0, split=-1: mx.mxgemm_plan(M, N, K, packed, split, 256)["kernel_name"]
    assert name(1, 1024, 2048) == "gemv_m1_n4"
    assert name(1, 1021, 2048) == "gemv_m1_n4"  # 256 workgroups, the last with one row
    assert name(1, 1020, 2048) != "gemv_m1_n4"
    assert name(1, 8192, 9216) != "gemv_m1_n4"
    assert name(1, 8192, 8192, packed=1) != "gemv_m1_n4"
    assert name(1, 8192, 8192, split=1) == "gemv_m1_n4"
    assert name(1, 8192, 8192, split=2) != "gemv_m1_n4"
    for M in (2, 3, 4, 5, 8):  # the small-batch forms, FP4 A
        assert name(M, 8192, 8192) == ("gemv_m4_n4" if M <= 4 else "gemv_m8_n4")
        assert mx.mxgemm_plan(M, 8192, 8192, 0, -1, 256)["tile_m"] == M
    assert name(9, 8192, 8192).startswith("skinny")
    assert mx.mxgemm_plan(1, 8192, 8192, 0, -1, 128)["grid"] == 2048
    for fmt in (mx.FMT_FP8_E4M3, mx.FMT_FP8_E5M2, mx.FMT_FP6_E2M3, mx.FMT_FP6_E3M2):
        st = mx.make_strides(ldd=8192, ldc=8192, lda=8192, ldb=8192, ldsa=256, ldsb=256, a_format=fmt)
        assert mx.mxgemm_plan_ex(1, 8192, 8192, st, -1, 256)["kernel_name"] == "gemv_m1_n4"
        assert mx.mxgemm_plan_ex(2, 8192, 8192, st, -1, 256)["kernel_name"].startswith("skinny")

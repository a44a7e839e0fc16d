#!/usr/bin/env python3
"""MXFP4 block-scaled GEMM benchmark on one MI355X (gfx950).

One step = one mxgemm_run call, i.e. the whole GEMM path (tile/split choice,
operand streaming, scaled FP4 matrix instructions, split-K reduction when
planned, fused alpha/beta bf16 epilogue) over one set of synthetic inputs
already resident in HBM.  The B pre-shuffle (mxgemm_pack_b) is per-weight
preparation and runs before timing, for the workload that uses it.

Headline line: the 8192^3 workload (packed B), TFLOP/s = 2MNK / time, with
the roofline of its kernel against the MI355X dense MXFP4 peak; the M = 1
decode workload is reported next to it in GB/s against HBM, and the other
workloads in a list.  Steps are launched from a HIP graph (captured once,
replayed) so that kernel-launch overhead of the Python caller does not show
up as GPU idle time; every kernel in the graph is a real mxgemm_run launch.
For HBM-bound workloads the inputs rotate over enough copies that each
step's operands are not resident in the last-level cache.  Before each
workload's timed replay the GPU runs 500 ms of untimed launches of the same
workload (--soak-ms), so that the timing sees the clock the chip settles at
under sustained load rather than its first-launch transient.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP4 GEMM TFLOPS (2MNK/s) + % of MXFP4 MFMA peak; GB/s at M=1"
PEAK_MXFP4_TFLOPS = 10100.0  # MI355X dense MXFP4 matrix peak (published)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E (published)
PAGE_TFLOPS_8192 = 4245.0    # asm_f4gemm README, "Measured": 8192^3 on MI355X
LLC_BYTES = 256 << 20        # MI355X last-level (Infinity) cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(workload):
    """HBM bytes per launch from the committed counter runs (profiles/traffic.json),
    or None when the workload's kernel family has changed since those
    counters were taken (each entry carries the fingerprint of its family's
    sources)."""
    from block_scaled_precision_mxfp4_amd.kernel_hash import FAMILY_FILES, kernel_family_hash
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    w = t.get("workloads", {}).get(workload)
    if w is None or w.get("family") not in FAMILY_FILES or w.get("source_hash") != kernel_family_hash(w["family"]):
        return None
    return w["traffic_bytes"]


def algorithmic_bytes(M, N, K, beta, a_bits=4):
    b = M * K * a_bits // 8 + M * K // 32 + N * K // 2 + N * K // 32 + 2 * M * N
    if beta != 0.0:
        b += 2 * M * N
    return b


def workload_roofline(r):
    """The roofline of one timed workload: its algorithmic flops against the
    MXFP4 matrix peak where its arithmetic intensity is above the ridge point
    (peak flops / 8 TB/s), else its algorithmic bytes against HBM; traffic
    from the committed counter runs while they match the kernel sources."""
    intensity = 2.0 * r["M"] * r["N"] * r["K"] / r["algorithmic_bytes"]
    if intensity >= PEAK_MXFP4_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        return {"bound": "mfma", "achieved": r["tflops"], "peak": PEAK_MXFP4_TFLOPS, "unit": "TFLOP/s",
                "frac": r["tflops"] / PEAK_MXFP4_TFLOPS, "traffic": measured_traffic(r["workload"])}
    return {"bound": "hbm", "achieved": r["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": r["gbs"] / PEAK_HBM_GBS, "traffic": measured_traffic(r["workload"])}


def time_workload(name, steps, warmup, split_k=-1, rotate=True, eager=False, soak_ms=0.0, a_fmt=0, b_layout=0,
                  packed=None, a_packed=False):
    import numpy as np
    import torch

    import block_scaled_precision_mxfp4_amd as mx
    from block_scaled_precision_mxfp4_amd import inputs

    p = inputs.make_workload(name)
    M, N, K, alpha, beta = p["M"], p["N"], p["K"], p["alpha"], p["beta"]
    sa_packed = p["sa_packed"]
    if packed is None:
        packed = p["b_packed"]
    elif packed and not sa_packed and M > 64:
        sa_packed = True
    ldb = K
    if b_layout:  # the same B stored MN-major ([K][N] codes), scales packed as the workload's
        p["B"] = inputs.to_mn_major(p["B"], N, K, N)
        ldb = N
    a_bits = mx.FORMAT_BITS[a_fmt]
    if a_fmt:  # the same workload with A in a wider format (row-major A scales)
        p["A"] = inputs.wide_codes(inputs.SEED_BASE + 0x100 + a_fmt, M, K, a_fmt)
        sa_packed = False
    if a_fmt or b_layout:
        info = mx.mxgemm_query_ex(M, N, K, mx.make_strides(ldd=N, ldc=N, lda=K, ldb=ldb, ldsa=K // 32, ldsb=K // 32,
                                                          b_packed=int(packed), sa_packed=int(sa_packed),
                                                          a_format=a_fmt, b_layout=b_layout,
                                                          a_packed=int(a_packed)), split_k)
        info["packed_b_bytes"] = mx.mxgemm_query(M, N, K, int(packed), split_k)["packed_b_bytes"]
        info["packed_sb_bytes"] = mx.mxgemm_query(M, N, K, int(packed), split_k)["packed_sb_bytes"]
    else:
        info = mx.mxgemm_query(M, N, K, int(packed), split_k)
    ws_bytes = algorithmic_bytes(M, N, K, beta, a_bits)
    copies = 1
    if rotate and ws_bytes < 2 * LLC_BYTES:
        copies = min(64, math.ceil(2.5 * LLC_BYTES / ws_bytes))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    A0, SA0, B0, SB0 = dev(p["A"]), dev(p["SA"]), dev(p["B"]), dev(p["SB"])
    C0 = None
    if p["C"] is not None:
        C0 = torch.from_numpy(p["C"].view(np.int16)).cuda().view(torch.bfloat16)
    sets = []
    for c in range(copies):
        A, SA = A0.clone(), SA0.clone()
        B, SB = B0.clone(), SB0.clone()
        C = C0.clone() if C0 is not None else None
        D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        if packed and b_layout:  # MN-major codes stay as they are; only the scales are shuffled
            SBp = torch.empty(info["packed_sb_bytes"], dtype=torch.uint8, device="cuda")
            mx.mxgemm_pack_scales(SBp, SB, N, K)
            SB = SBp
        elif packed:
            Bp = torch.empty(info["packed_b_bytes"], dtype=torch.uint8, device="cuda")
            SBp = torch.empty(info["packed_sb_bytes"], dtype=torch.uint8, device="cuda")
            mx.mxgemm_pack_b(Bp, SBp, B, SB, N, K)
            B, SB = Bp, SBp
        if sa_packed:
            SAp = torch.empty(info["packed_sa_bytes"], dtype=torch.uint8, device="cuda")
            mx.mxgemm_pack_scales(SAp, SA, M, K)
            SA = SAp
        if a_packed:  # FP6 A and its scales put into the dense tile's order once, like a packed B
            Ap = torch.empty(mx.mxgemm_pack_a_bytes(M, K), dtype=torch.uint8, device="cuda")
            SAp = torch.empty(info["packed_sa_bytes"], dtype=torch.uint8, device="cuda")
            mx.mxgemm_pack_a(Ap, SAp, A, SA, M, K, a_fmt)
            A, SA = Ap, SAp
        sets.append((D, C, A, B, SA, SB))
    del A0, SA0, B0, SB0, C0
    wsp = torch.zeros(max(info["workspace_bytes"], 256), dtype=torch.uint8, device="cuda")
    strides = mx.make_strides(ldd=N, ldc=N, lda=K, ldb=ldb, ldsa=K // 32, ldsb=K // 32,
                              b_packed=int(packed), sa_packed=int(sa_packed), workspace=wsp,
                              workspace_bytes=wsp.numel(), a_format=a_fmt, b_layout=b_layout,
                              a_packed=int(a_packed))
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()

    def launch(i):
        D, C, A, B, SA, SB = sets[i % copies]
        mx.mxgemm_run(D, C if beta != 0.0 else None, A, B, SA, SB, alpha, beta, M, N, K,
                      strides=strides, split_k=split_k, stream=stream.cuda_stream)

    with torch.cuda.stream(stream):
        for i in range(warmup):
            launch(i)
    torch.cuda.synchronize()
    if soak_ms > 0:
        # untimed load until the clocks have settled (the chip lowers its
        # clock under sustained matrix load): sustained, not burst, speed
        t_end = time.perf_counter() + soak_ms / 1e3
        i = 0
        while time.perf_counter() < t_end:
            with torch.cuda.stream(stream):
                for _ in range(64):
                    launch(i)
                    i += 1
            stream.synchronize()

    timing = "hipgraph"
    graph = None
    if eager:
        timing = "eager"
    try:
        if eager:
            raise RuntimeError("eager launches requested")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                launch(i)
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
    except Exception as e:  # capture unsupported: fall back to eager launches
        log("graph capture failed (%s); timing eager launches" % e)
        graph, timing = None, "eager"

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):  # the graph replays on the current stream
        e0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(steps):
                launch(i)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    per = gpu_ms / 1e3 / steps
    flops = 2.0 * M * N * K
    r = dict(workload=name, a_format=a_fmt, b_layout=("kn" if b_layout else "nk"), M=M, N=N, K=K, alpha=alpha,
             beta=beta, b_packed=bool(packed),
             sa_packed=bool(sa_packed),
             kernel=info["kernel_name"], tile="%dx%d" % (info["tile_m"], info["tile_n"]),
             split_k=info["split_k"], grid=info["grid"], copies=copies, timing=timing,
             us_per_step=per * 1e6, tflops=flops / per / 1e12,
             gbs=algorithmic_bytes(M, N, K, beta, a_bits) / per / 1e9,
             algorithmic_bytes=algorithmic_bytes(M, N, K, beta, a_bits), wall_s=wall, gpu_ms=gpu_ms,
             peak_flops_device=info["peak_flops"], clock_hz=info["clock_hz"], num_cu=info["num_cu"],
             arch=info["arch"])
    del sets, wsp
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log("%-24s %-22s split %2d  %9.2f us  %8.1f TFLOP/s  %8.1f GB/s  (%s, %d copies)" % (
        name + ("" if not a_fmt else " A:" + FORMAT_NAMES[a_fmt]) + (" B:KN" if b_layout else "") +
        (" packed" if packed and not p["b_packed"] else ""), r["kernel"], r["split_k"], r["us_per_step"],
        r["tflops"], r["gbs"], timing, copies))
    return r


PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak


def time_f16(steps, warmup, soak_ms=0.0, M=8192, N=8192, K=8192):
    """mxgemm_f16_run (fp32 C = fp16 A x K-major fp16 B) on one 8192^3
    problem, HIP-graph replay (operands stay in HBM and the last-level
    cache between steps, as for the square MXFP4 workload)."""
    import torch

    import block_scaled_precision_mxfp4_amd as mx

    g = torch.Generator(device="cuda").manual_seed(0xF16)
    A = torch.randn((M, K), device="cuda", generator=g).to(torch.float16)
    B = torch.randn((K, N), device="cuda", generator=g).to(torch.float16)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def launch():
        mx.mxgemm_f16_run(C, A, B, M, N, K, stream=stream.cuda_stream)

    with torch.cuda.stream(stream):
        for _ in range(warmup):
            launch()
    torch.cuda.synchronize()
    if soak_ms > 0:
        t_end = time.perf_counter() + soak_ms / 1e3
        while time.perf_counter() < t_end:
            with torch.cuda.stream(stream):
                for _ in range(16):
                    launch()
            stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(steps):
            launch()
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    per = e0.elapsed_time(e1) / 1e3 / steps
    tflops = 2.0 * M * N * K / per / 1e12
    log("%-24s %-22s           %9.2f us  %8.1f TFLOP/s  (hipgraph)" % ("f16_8192", "mx_f16_kernel", per * 1e6, tflops))
    return {"workload": "f16_%dx%dx%d" % (M, N, K), "us_per_step": per * 1e6, "value": tflops, "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                         "frac": tflops / PEAK_F16_TFLOPS, "traffic": None}}


FORMAT_NAMES = {0: "fp4", 1: "fp8_e4m3", 2: "fp8_e5m2", 3: "fp6_e2m3", 4: "fp6_e3m2"}
FORMAT_CODES = {v: k for k, v in FORMAT_NAMES.items()}
# mixed-format lines: (workload, A format) -- decode and a small batch with
# FP8 and FP6 activations against FP4 weights
MIXED = [("gemv_1x8192x8192", 1), ("gemv_1x8192x8192", 3), ("skinny_64x7168x16384", 1), ("square_8192", 1),
         ("skinny_64x7168x16384", 3), ("square_8192", 3)]
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense 8-bit scaled matrix peak (half the FP4 rate)

QUANT_SHAPE = (8192, 8192)  # the bf16 activation of the square workload's A


def quant_bytes(M, K):
    """Algorithmic bytes of one quantizer call: bf16 in, fp4x2 codes and one
    scale byte per 32 elements out."""
    return 2 * M * K + M * K // 2 + M * K // 32


def time_decode(steps, warmup, soak_ms=0.0, N=8192, K=8192):
    """The decode step 1 x N x K from a bf16 activation: mxgemm_run_bf16a (the
    quantizer fused into the GEMV's A load, one launch) against
    mxgemm_quantize followed by mxgemm_run (two launches), each HIP-graph
    replayed over rotated B copies so that B comes from HBM."""
    import torch

    import block_scaled_precision_mxfp4_amd as mx

    copies = max(1, math.ceil(2.5 * LLC_BYTES / (N * K // 2 + N * K // 32)))
    g = torch.Generator(device="cuda").manual_seed(0xDEC)
    X = torch.randn((1, K), device="cuda", generator=g).to(torch.bfloat16)
    Bs = [(torch.randint(0, 256, (N, K // 2), device="cuda", dtype=torch.uint8, generator=g),
           torch.randint(118, 136, (N, K // 32), device="cuda", dtype=torch.uint8, generator=g))
          for _ in range(copies)]
    A = torch.empty((1, K // 2), dtype=torch.uint8, device="cuda")
    SA = torch.empty((1, K // 32), dtype=torch.uint8, device="cuda")
    D = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.Stream()
    cs = stream.cuda_stream

    def fused(i):
        B, SB = Bs[i % copies]
        mx.mxgemm_run_bf16a(D, None, X, B, SB, 1.0, 0.0, 1, N, K, stream=cs)

    def two_step(i):
        B, SB = Bs[i % copies]
        mx.mxgemm_quantize(A, SA, X, 1, K, stream=cs)
        mx.mxgemm_run(D, None, A, B, SA, SB, 1.0, 0.0, 1, N, K, stream=cs)

    out = {}
    for name, launch in (("fused", fused), ("quantize_then_gemm", two_step)):
        with torch.cuda.stream(stream):
            for i in range(warmup):
                launch(i)
            if soak_ms > 0:
                t_end = time.time() + soak_ms / 1e3
                i = 0
                while time.time() < t_end:
                    launch(i)
                    i += 1
                    if i % 64 == 0:
                        torch.cuda.synchronize()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                launch(i)
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) * 1e3 / steps
        del graph
    log("%-24s %-22s           %9.2f us  (quantize then GEMM: %.2f us, hipgraph, %d copies)" % (
        "decode_1x%dx%d" % (N, K), "fused bf16 A", out["fused"], out["quantize_then_gemm"], copies))
    return {"workload": "decode_1x%dx%d_bf16_activation" % (N, K), "us_per_step": out["fused"],
            "us_two_launches": out["quantize_then_gemm"], "copies": copies}


def time_quantize(steps, warmup, eager=False):
    """mxgemm_quantize on QUANT_SHAPE, HIP-graph replay over rotated inputs."""
    import torch

    import block_scaled_precision_mxfp4_amd as mx

    M, K = QUANT_SHAPE
    nbytes = quant_bytes(M, K)
    copies = max(1, math.ceil(2.5 * LLC_BYTES / nbytes))
    g = torch.Generator(device="cuda").manual_seed(0x5EED)
    sets = []
    for _ in range(copies):
        X = (torch.randn((M, K), device="cuda", generator=g) *
             torch.exp2(torch.randint(-20, 20, (M, 1), device="cuda", generator=g).float())).to(torch.bfloat16)
        A = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
        S = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
        sets.append((A, S, X))
    stream = torch.cuda.Stream()
    launch = lambda i: mx.mxgemm_quantize(*sets[i % copies], M, K, stream=stream.cuda_stream)
    with torch.cuda.stream(stream):
        for i in range(warmup):
            launch(i)
    torch.cuda.synchronize()
    graph, timing = None, "eager"
    if not eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                launch(i)
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        timing = "hipgraph"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(steps):
                launch(i)
        e1.record(stream)
    torch.cuda.synchronize()
    per = e0.elapsed_time(e1) / 1e3 / steps
    gbs = nbytes / per / 1e9
    del sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log("%-24s %-22s          %9.2f us  %8.1f GB/s  (%s, %d copies)" % (
        "quantize_%dx%d" % (M, K), "mx_quant_kernel", per * 1e6, gbs, timing, copies))
    return {"workload": "quantize_%dx%d" % (M, K), "value": gbs, "unit": "GB/s",
            "us_per_step": per * 1e6, "algorithmic_bytes": nbytes, "copies": copies, "timing": timing,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS,
                         "traffic": measured_traffic("quantize_%dx%d" % (M, K))}}


def time_stream_read(nbytes, steps, warmup):
    """mxgemm_stream_read of nbytes over rotated copies (as many as the GEMM
    lines rotate for that byte count), HIP-graph replay: the HBM read rate
    this chip reaches for a kernel whose minimum traffic is nbytes."""
    import torch

    import block_scaled_precision_mxfp4_amd as mx

    nbytes = nbytes // 16 * 16
    copies = max(1, math.ceil(2.5 * LLC_BYTES / nbytes))
    g = torch.Generator(device="cuda").manual_seed(0x57EA)
    bufs = [torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g) for _ in range(copies)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    launch = lambda i: mx.mxgemm_stream_read(bufs[i % copies], nbytes, sink, stream=stream.cuda_stream)
    with torch.cuda.stream(stream):
        for i in range(warmup):
            launch(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            launch(i)
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    per = e0.elapsed_time(e1) / 1e3 / steps
    del bufs, graph
    torch.cuda.empty_cache()
    gbs = nbytes / per / 1e9
    log("%-24s %-22s           %9.2f us  %8.1f GB/s  (hipgraph, %d copies)" % (
        "stream_read_%d" % nbytes, "mx_stream_read_kernel", per * 1e6, gbs, copies))
    return {"bytes": nbytes, "us_per_step": per * 1e6, "gbs": gbs, "frac_of_peak": gbs / PEAK_HBM_GBS,
            "copies": copies}


def cpu_baseline(name, target_s=12.0):
    """The oracle, as it stands, on a bounded sample of the workload's outputs:
    threaded over the output columns (the machine's CPU share is 16 cores per GPU,
    whatever the host's own count), and on one thread for a 64-row slice."""
    import numpy as np

    import oracle
    from block_scaled_precision_mxfp4_amd import inputs

    p = inputs.make_workload(name)
    M, N, K = p["M"], p["N"], p["K"]
    threads = max(1, min(16, os.cpu_count() or 1))
    # grow the sample (whole rows of the output, capped by its size) until a
    # run takes a sizeable fraction of target_s, then scale it to target_s
    n_cols = min(N, 1024)
    n_rows = 1
    while True:
        rows = np.arange(n_rows, dtype=np.int64)
        cols = np.arange(n_cols, dtype=np.int64)
        t0 = time.perf_counter()
        oracle.mxgemm(p["A"], p["SA"], p["B"], p["SB"], K, p["alpha"], p["beta"], p["C"],
                      rows=rows, cols=cols, threads=threads)
        dt = time.perf_counter() - t0
        if dt >= target_s / 3 or n_rows * n_cols >= M * N:
            break
        grow = min(8.0, max(2.0, target_s / max(dt, 1e-3)))
        if n_cols < N:
            n_cols = min(N, int(n_cols * grow))
        else:
            n_rows = min(M, max(n_rows + 1, int(n_rows * grow)))
    macs = n_rows * n_cols * K
    # one thread: a 64-row slice of the first 64 columns, extrapolated to the
    # whole workload at the same per-MAC rate
    rows1 = np.arange(min(M, 64), dtype=np.int64)
    cols1 = np.arange(min(N, 64), dtype=np.int64)
    t0 = time.perf_counter()
    oracle.mxgemm(p["A"], p["SA"], p["B"], p["SB"], K, p["alpha"], p["beta"], p["C"],
                  rows=rows1, cols=cols1, threads=1)
    dt1 = time.perf_counter() - t0
    macs1 = len(rows1) * len(cols1) * K
    return {"value": 2.0 * macs / dt / 1e9, "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(),
            "sample": "%d rows x %d cols of %s (%.3g MACs, fp64) in %.2f s on %d threads" % (
                n_rows, n_cols, name, macs, dt, threads),
            "single_thread": {"value": 2.0 * macs1 / dt1 / 1e9, "unit": "GFLOP/s", "cores": 1,
                              "sample": "%d rows x %d cols of %s (%.3g MACs) in %.2f s" % (
                                  len(rows1), len(cols1), name, macs1, dt1),
                              "extrapolated_full_s": dt1 * (M * N * K) / macs1}}


def tile_split_sweep(name, args):
    """The workload on every tile shape (forced) at splits 1, 2 and 4: us per
    step (checks the planner's pick, timed on its own line)."""
    import block_scaled_precision_mxfp4_amd as mx
    out = []
    n_tiles = 4
    for tile in range(n_tiles):
        os.environ["MXGEMM_FORCE_TILE"] = str(tile)
        try:
            for s in (1, 2, 4):
                r = time_workload(name, args.steps, args.warmup, split_k=s, eager=args.eager,
                                  soak_ms=min(args.soak_ms, 100.0))
                out.append({"tile": r["tile"], "kernel": r["kernel"], "split_k": r["split_k"],
                            "us_per_step": r["us_per_step"]})
        finally:
            del os.environ["MXGEMM_FORCE_TILE"]
    return out


def split_sweep(name, args):
    """The workload at every forced split (the heuristic's pick is timed on
    its own line): us and algorithmic GB/s per split."""
    out = []
    for s in (1, 2, 4, 8, 16):
        r = time_workload(name, args.steps, args.warmup, split_k=s, eager=args.eager,
                          soak_ms=min(args.soak_ms, 100.0))
        out.append({"split_k": r["split_k"], "us_per_step": r["us_per_step"], "gbs": r["gbs"]})
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="square_8192")
    ap.add_argument("--split-k", type=int, default=-1)
    ap.add_argument("--only", action="store_true", help="time only --workload (profiling runs)")
    ap.add_argument("--b-layout", choices=("nk", "kn"), default="nk",
                    help="B of --workload stored K-major (nk, the default) or MN-major (kn, scales packed)")
    ap.add_argument("--packed", action="store_true", help="pre-shuffle B of --workload (and A scales if M > 64)")
    ap.add_argument("--a-packed", action="store_true",
                    help="FP6 A of --workload put into the dense tile's order once (mxgemm_pack_a; profiling runs)")
    ap.add_argument("--a-format", choices=sorted(FORMAT_CODES), default="fp4",
                    help="A of --workload in this format (profiling runs of the mixed-format lines)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch steps one by one (counter runs)")
    ap.add_argument("--soak-ms", type=float, default=500.0,
                    help="untimed load before each workload's timing, so that the clocks have "
                         "settled (0: time right after the warmup launches)")
    ap.add_argument("--quantize-only", action="store_true",
                    help="time only the bf16 -> MXFP4 quantizer (profiling runs)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, 5 times (counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the GEMM runs on a single MI355X and this build has "
              "no multi-GPU path (requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_precision_mxfp4_amd as mx
    from block_scaled_precision_mxfp4_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.calib_copy:
        src = torch.randint(0, 255, (args.calib_copy,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": args.calib_copy, "copies": 5}), flush=True)
        return
    mx.lib()
    if args.quantize_only:
        print(json.dumps(time_quantize(args.steps, args.warmup, eager=args.eager)), flush=True)
        return

    head = time_workload(args.workload, args.steps, args.warmup, split_k=args.split_k, eager=args.eager,
                         soak_ms=args.soak_ms, b_layout=int(args.b_layout == "kn"),
                         packed=True if (args.b_layout == "kn" or args.packed) else None,
                         a_fmt=FORMAT_CODES[args.a_format], a_packed=args.a_packed)
    others = []
    if not args.only:
        for name in inputs.WORKLOADS:
            if name != args.workload:
                others.append(time_workload(name, args.steps, args.warmup, eager=args.eager,
                                            soak_ms=args.soak_ms))
    gemv = next((o for o in [head] + others if o["M"] == 1), None)

    m1 = None
    if gemv is not None:
        m1 = {"workload": gemv["workload"], "value": gemv["gbs"], "unit": "GB/s",
              "us_per_step": gemv["us_per_step"], "split_k": gemv["split_k"],
              "algorithmic_bytes": gemv["algorithmic_bytes"],
              "roofline": {"bound": "hbm", "achieved": gemv["gbs"], "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": gemv["gbs"] / PEAK_HBM_GBS,
                           "traffic": measured_traffic(gemv["workload"])}}
        if not args.only:
            m1["split_sweep"] = split_sweep(gemv["workload"], args)

    if m1 is not None and not args.eager:
        # the achievable HBM read rate for the same byte count, rotated the same way
        st = time_stream_read(gemv["algorithmic_bytes"], args.steps, args.warmup)
        m1["achievable_gbs"] = st["gbs"]
        m1["stream_read"] = st
        m1["frac_of_achievable"] = gemv["gbs"] / st["gbs"]

    quant = None if args.only else time_quantize(args.steps, args.warmup, eager=args.eager)
    decode = None if args.only or args.eager else time_decode(args.steps, args.warmup, soak_ms=min(args.soak_ms, 200.0))

    f16 = None if args.only else time_f16(args.steps, args.warmup, soak_ms=args.soak_ms)

    mixed = []
    if not args.only:
        # (the last entry: the FP6 square with A put into the dense tile's
        # order once by mxgemm_pack_a, outside the timed call, as B is)
        for name, fmt, a_packed in [(n, f, False) for n, f in MIXED] + [("square_8192", 3, True)]:
            r = time_workload(name, args.steps, args.warmup, eager=args.eager, soak_ms=args.soak_ms, a_fmt=fmt,
                              a_packed=a_packed)
            if r["M"] > 64:  # a contraction: the matrix peak of A's format (FP6 runs at the FP4 rate)
                peak = PEAK_FP8_TFLOPS if fmt in (1, 2) else PEAK_MXFP4_TFLOPS
                roof = {"bound": "mfma", "achieved": r["tflops"], "peak": peak, "unit": "TFLOP/s",
                        "frac": r["tflops"] / peak,
                        "traffic": measured_traffic(name + "_" + FORMAT_NAMES[fmt] + ("_packed_a" if a_packed else ""))}
                value, unit = r["tflops"], "TFLOP/s"
            else:
                roof = {"bound": "hbm", "achieved": r["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": r["gbs"] / PEAK_HBM_GBS, "traffic": measured_traffic(name + "_" + FORMAT_NAMES[fmt])}
                value, unit = r["gbs"], "GB/s"
            mixed.append({"workload": name, "a_format": FORMAT_NAMES[fmt], "a_packed": a_packed,
                          "us_per_step": r["us_per_step"],
                          "value": value, "unit": unit, "tflops": r["tflops"],
                          "algorithmic_bytes": r["algorithmic_bytes"], "kernel": r["kernel"], "roofline": roof})

    # B stored MN-major ([K][N], read through the transposed LDS loads) on
    # the square workload, and the skinny workload with a pre-shuffled B
    layouts = []
    if not args.only:
        for name, b_layout, packed in (("square_8192", 1, True), ("skinny_64x7168x16384", 0, True)):
            r = time_workload(name, args.steps, args.warmup, eager=args.eager, soak_ms=args.soak_ms,
                              b_layout=b_layout, packed=packed)
            key = name + ("_kn" if b_layout else "_packed")
            if r["M"] > 64:
                roof = {"bound": "mfma", "achieved": r["tflops"], "peak": PEAK_MXFP4_TFLOPS, "unit": "TFLOP/s",
                        "frac": r["tflops"] / PEAK_MXFP4_TFLOPS, "traffic": measured_traffic(key)}
            else:
                roof = {"bound": "hbm", "achieved": r["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": r["gbs"] / PEAK_HBM_GBS, "traffic": measured_traffic(key)}
            layouts.append({"workload": name, "b_layout": r["b_layout"], "b_packed": r["b_packed"],
                            "sa_packed": r["sa_packed"], "kernel": r["kernel"], "tile": r["tile"],
                            "split_k": r["split_k"], "us_per_step": r["us_per_step"], "tflops": r["tflops"],
                            "gbs": r["gbs"], "roofline": roof})

    base = None
    if not args.no_cpu_baseline:
        base = cpu_baseline(args.workload)
        log("cpu baseline:", base)

    hbm_bound = head["M"] <= 64
    if hbm_bound:
        value, unit = head["gbs"], "GB/s"
        roof = {"bound": "hbm", "achieved": head["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": head["gbs"] / PEAK_HBM_GBS, "traffic": measured_traffic(head["workload"])}
    else:
        value, unit = head["tflops"], "TFLOP/s"
        roof = {"bound": "mfma", "achieved": head["tflops"], "peak": PEAK_MXFP4_TFLOPS,
                "unit": "TFLOP/s", "frac": head["tflops"] / PEAK_MXFP4_TFLOPS,
                "traffic": measured_traffic(head["workload"]),
                "algorithmic_bytes": head["algorithmic_bytes"]}
    vs = value / PAGE_TFLOPS_8192 if head["workload"] == "square_8192" and unit == "TFLOP/s" else None
    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["us_per_step"] / 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": vs, "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": head["workload"], "M": head["M"], "N": head["N"], "K": head["K"],
                   "b_packed": head["b_packed"], "sa_packed": head["sa_packed"], "kernel": head["kernel"],
                   "tile": head["tile"],
                   "split_k": head["split_k"], "timing": head["timing"]},
        "roofline": roof,
        "cpu_baseline": base,
        "m1": m1,
        "mixed": mixed,
        "f16": f16,
        "quantize": quant,
        "decode": decode,
        "b_layouts": layouts,
        "device": {"arch": head["arch"], "num_cu": head["num_cu"], "clock_hz": head["clock_hz"],
                   "derived_peak_tflops": head["peak_flops_device"] / 1e12},
        "workloads": [dict({k: o[k] for k in ("workload", "kernel", "tile", "split_k", "us_per_step",
                                              "tflops", "gbs", "copies", "timing")},
                           roofline=workload_roofline(o)) for o in [head] + others],
    }
    skinny = next((o for o in others if o["workload"] == "skinny_64x7168x16384"), None)
    if skinny is not None:
        line["skinny_split_sweep"] = split_sweep(skinny["workload"], args)
    mid = next((o for o in others if o["workload"] == "mid_512x1024x2048"), None)
    if mid is not None:
        line["mid_tile_split_sweep"] = tile_split_sweep(mid["workload"], args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

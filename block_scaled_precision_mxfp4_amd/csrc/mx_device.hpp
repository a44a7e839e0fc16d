// Device-side building blocks shared by the MXFP4 GEMM kernels (gfx950).
//
// Operand fragments.  The 16x16x128 scaled matrix instruction ("CDNA4 dense
// MFMA builtins", section "Mixed-precision with scaling") takes, for FP4
// (format selector 4), 32 E2M1 values per lane: lane l holds row l % 16 of
// its operand and the 32 consecutive K elements of K-block l / 16, i.e. 16
// bytes.  One such fragment is therefore exactly 16 rows x 128 K = 1 KiB,
// and "lane-linear" 1 KiB chunks (lane l's 16 bytes at offset 16*l) are the
// unit in which the kernels move operands: it is also the unit of the
// 16x16 tile-transposed B layout of the asm_f4gemm README ("Data layouts").
// Each lane passes one 32-bit scale register per operand; the 2-bit op_sel
// immediate picks which of its four E8M0 bytes applies to that lane's
// K-block.
//
// Result layout ("CDNA4 dense MFMA builtins", "Accumulator layout", 16x16):
// lane l, accumulator g holds row 4*(l/16) + g, column l % 16.  The kernels
// feed B as the instruction's first operand and A as its second, so the
// instruction's rows are columns n of D and its columns are rows m of D:
// every lane ends up with four consecutive n of one row m.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

// Format selector of E2M1 for the scaled matrix instructions (the fifth
// entry of the format table, codes 0..4).
constexpr int kFmtFp4 = 4;
// Buffer-resource word 3 for gfx9-family raw buffers (no swizzle, range
// checked against num_records).
constexpr int kRsrcWord3 = 0x00020000;
// A byte offset that is always outside any buffer resource's range: loads
// from it return zero and do not touch memory.
constexpr uint32_t kOOB = 0xFFFFFF00u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// make_rsrc for values the compiler cannot prove wave-uniform (e.g. after an
// integer division, which is computed in vector registers): without the
// explicit read-first-lane every buffer access through the descriptor
// becomes a loop over the distinct descriptors of the lanes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_u(const void *base, uint32_t bytes)
{
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return make_rsrc((const void *)(uintptr_t)(((uint64_t)hi << 32) | lo), n);
}

__device__ __forceinline__ v4i load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ v2u load8(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t load1(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// 16 bytes per lane straight from global memory into LDS at lds + 16*lane
// (lds must be wave-uniform).  Out-of-range lanes write zeros.
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t r, lds_void *lds, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, off, 0, 0, 0);
}

// Transposed 4-bit LDS read ("CDNA4 MFMA transpose load builtins",
// ds_read_tr4_b64): within each group of 16 lanes, lane q names 8 bytes (16
// codes, element j in nibble j) and lane j receives code j of every lane q
// of its group, in nibble q.  p must point into LDS, 8-byte aligned.
__device__ __forceinline__ v2i lds_tr4(const uint8_t *p)
{
    return __builtin_amdgcn_ds_read_tr4_b64_v2i32((__attribute__((address_space(3))) v2i *)(p));
}

// Cache policy of operands that are read once per call (the B stream of the
// skinny kernels): the non-temporal hint (nt) asks the caches not to keep
// the lines.
constexpr int kStream = 2;

__device__ __forceinline__ void load16_to_lds_stream(__amdgpu_buffer_rsrc_t r, lds_void *lds, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, off, 0, 0, kStream);
}

__device__ __forceinline__ v4i load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStream);
}

// acc += (B fragment, scaled) x (A fragment, scaled) over 128 K.
template <int OPSEL_B, int OPSEL_A>
__device__ __forceinline__ v4f mfma_fp4(v4i bfrag, v4i afrag, v4f acc, int sb, int sa)
{
    v8i b = {bfrag[0], bfrag[1], bfrag[2], bfrag[3], 0, 0, 0, 0};
    v8i a = {afrag[0], afrag[1], afrag[2], afrag[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, acc, kFmtFp4, kFmtFp4,
                                                           OPSEL_B, sb, OPSEL_A, sa);
}

// op_sel must be an immediate: select among the 16 (B byte, A byte) forms.
// With fully unrolled loops the selector is a constant and the switch folds.
__device__ __forceinline__ v4f mma_sel(int ob, int oa, v4i b, v4i a, v4f c, int sb, int sa)
{
#define MX_CASE(OB, OA) \
    case OB * 4 + OA: return mfma_fp4<OB, OA>(b, a, c, sb, sa);
    switch (ob * 4 + oa) {
        MX_CASE(0, 0) MX_CASE(0, 1) MX_CASE(0, 2) MX_CASE(0, 3)
        MX_CASE(1, 0) MX_CASE(1, 1) MX_CASE(1, 2) MX_CASE(1, 3)
        MX_CASE(2, 0) MX_CASE(2, 1) MX_CASE(2, 2) MX_CASE(2, 3)
        MX_CASE(3, 0) MX_CASE(3, 1) MX_CASE(3, 2) MX_CASE(3, 3)
    }
#undef MX_CASE
    return c;
}

// A operand of a wider format (FP8 E4M3 / BF8 E5M2: 8 dwords; FP6 E2M3 /
// E3M2: the low 6 dwords), B FP4: the hardware format code of A (the
// instruction's "blgp", since B is the instruction's first source) selects
// the element type ("CDNA4 dense MFMA builtins", "Mixed-precision with
// scaling": codes 0 FP8, 1 BF8, 2 FP6 E2M3, 3 FP6 E3M2, 4 FP4).
template <int FMT_A, int OPSEL_B, int OPSEL_A>
__device__ __forceinline__ v4f mfma_fp4_wide(v4i bfrag, v8i afrag, v4f acc, int sb, int sa)
{
    v8i b = {bfrag[0], bfrag[1], bfrag[2], bfrag[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, afrag, acc, kFmtFp4, FMT_A, OPSEL_B, sb,
                                                           OPSEL_A, sa);
}

template <int FMT_A>
__device__ __forceinline__ v4f mma_sel_wide(int ob, int oa, v4i b, v8i a, v4f c, int sb, int sa)
{
#define MX_CASE(OB, OA) \
    case OB * 4 + OA: return mfma_fp4_wide<FMT_A, OB, OA>(b, a, c, sb, sa);
    switch (ob * 4 + oa) {
        MX_CASE(0, 0) MX_CASE(0, 1) MX_CASE(0, 2) MX_CASE(0, 3)
        MX_CASE(1, 0) MX_CASE(1, 1) MX_CASE(1, 2) MX_CASE(1, 3)
        MX_CASE(2, 0) MX_CASE(2, 1) MX_CASE(2, 2) MX_CASE(2, 3)
        MX_CASE(3, 0) MX_CASE(3, 1) MX_CASE(3, 2) MX_CASE(3, 3)
    }
#undef MX_CASE
    return c;
}

// A formats, the library's ids (mxgemm_strides.a_format): element width and
// the matrix instruction's format code
constexpr int kFmtBits[5] = {4, 8, 8, 6, 6};
constexpr int kFmtHw[5] = {4, 0, 1, 2, 3};

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN (quiet).
// Two floats to two bf16 (round to nearest even) packed low/high: one
// v_cvt_pk_bf16_f32, which rounds with the wave's mode (nearest even, fp32
// denormals preserved -- the kernel descriptor's defaults) and returns a
// quiet NaN for a NaN input.  A software rounding (add 0x7FFF + lsb, NaN
// test) compiled to a divergent branch per value.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi)
{
    typedef float v2f_t __attribute__((ext_vector_type(2)));
    typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
    const v2f_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2bf_t));
}

__device__ __forceinline__ uint32_t bf16_rne(float f) { return bf16x2_rne(f, f) & 0xFFFFu; }

__device__ __forceinline__ float bf16_to_f32(uint32_t h)
{
    return __uint_as_float(h << 16);
}

// Scale bytes of 4 consecutive 128-K steps for one lane.  The lane's
// K-block within a step is lane/16; a row's 16 scale bytes for the 4 steps
// are contiguous.  The load and the packing into a register are separate
// steps: the packing (byte u = scale of step u, so op_sel = u picks it) runs
// only when the multiplies need the word, so waiting for the scale load never
// holds up the operand loads issued after it.  SVEC: one aligned 16-byte
// load per row (pitch and K-block count multiples of 16, so a group is
// entirely inside or outside the chunk); otherwise byte loads, blocks at or
// past kb_end reading as zero.
template <bool SVEC>
__device__ __forceinline__ v4i load_scale_raw(__amdgpu_buffer_rsrc_t r, int64_t ld, int row, int kb0, int kb_end,
                                              int lane)
{
    if constexpr (SVEC) {
        return load16(r, kb0 < kb_end ? (uint32_t)(row * ld + kb0) : kOOB);
    } else {
        const int j = lane >> 4;
        v4i w;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kb = kb0 + 4 * u + j;
            w[u] = (int)load1(r, kb < kb_end ? (uint32_t)(row * ld + kb) : kOOB);
        }
        return w;
    }
}

template <bool SVEC>
__device__ __forceinline__ uint32_t scale_group_word(v4i w, int lane)
{
    const int j = lane >> 4;
    uint32_t out = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t b = SVEC ? (((uint32_t)w[u] >> (8 * j)) & 0xFFu) : ((uint32_t)w[u] & 0xFFu);
        out |= b << (8 * u);
    }
    return out;
}

// Epilogue parameters shared by all kernels.
struct Epilogue {
    uint16_t *D;
    const void *C;  // bf16, or float32 when c_f32
    float alpha, beta;
    int M, N;
    int64_t ldd, ldc;
    int d_vec;  // D rows and base allow 8-byte stores of 4 consecutive n
    int c_vec;  // C rows and base allow one vector load of 4 consecutive n
    int c_f32;
};

// Epilogue for beta == 0 through a private LDS region of the wave
// (16*FM x 16*FN bf16, 16-byte chunks of a row XOR-swizzled by row / 2:
// with 8-byte writes served 32 lanes per cycle, rows r and r + 8 of the 16
// a write instruction covers must not share a slot; rows of 256 bytes (FN =
// 8) all start on bank 0 and are swizzled by row % 16 instead): the
// fragments are rounded and written to LDS in their own layout,
// then read back row-wise and written to D with 16-byte stores, each
// instruction covering whole 16*FN-column row segments (full 128-byte lines
// for FN = 4) instead of 32-byte pieces of 16 rows.  Same values as
// store_quad: one rounding of alpha*acc per element.  Needs D 16-byte
// aligned and ldd a multiple of 8; the wave must own `lds` exclusively.
template <int FM, int FN>
__device__ __forceinline__ void store_tile_staged(const Epilogue &ep, int m_base, int n_base,
                                                  const v4f (&acc)[FN][FM], uint8_t *lds)
{
    constexpr int RB = FN * 32;       // bytes per row of the wave tile
    constexpr int CH = RB / 16;       // 16-byte chunks per row (power of two)
    constexpr int RPI = 64 / CH;      // rows per copy-out instruction
    static_assert(CH == 2 || CH == 4 || CH == 8 || CH == 16, "row chunking");
    auto sw = [](int r) { return CH == 16 ? (r & 15) : ((r >> 1) & (CH - 1)); };
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int r = fm * 16 + (lane & 15);
            const int j = fn * 2 + (lane >> 5);
            v2u o;
            o[0] = bf16x2_rne(ep.alpha * acc[fn][fm][0], ep.alpha * acc[fn][fm][1]);
            o[1] = bf16x2_rne(ep.alpha * acc[fn][fm][2], ep.alpha * acc[fn][fm][3]);
            *reinterpret_cast<v2u *>(lds + r * RB + ((j ^ sw(r)) * 16) + ((lane >> 4) & 1) * 8) = o;
        }
#pragma unroll
    for (int i = 0; i < FM * 16 / RPI; ++i) {
        const int r = i * RPI + lane / CH, c = lane & (CH - 1);
        const v4i v = *reinterpret_cast<const v4i *>(lds + r * RB + ((c ^ sw(r)) * 16));
        const int m = m_base + r, n = n_base + c * 8;
        if (m >= ep.M || n >= ep.N)
            continue;
        uint16_t *drow = ep.D + (int64_t)m * ep.ldd + n;
        if (n + 7 < ep.N) {
            // D is written once and not read back here: streaming stores keep
            // it from displacing operand lines in L2
            __builtin_nontemporal_store(v, reinterpret_cast<v4i *>(drow));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < ep.N)
                    drow[e] = (uint16_t)(((uint32_t)v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        }
    }
}

// Writes D[m][n..n+3] = bf16(alpha*acc[g] + beta*C[m][n+g]) for the
// elements inside the matrix.  One rounding per element.
__device__ __forceinline__ void store_quad(const Epilogue &ep, int m, int n, v4f acc)
{
    if (m >= ep.M || n >= ep.N)
        return;
    float r[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
        r[g] = ep.alpha * acc[g];
    const bool full = n + 3 < ep.N;
    if (ep.beta != 0.0f && ep.c_f32) {
        const float *crow = reinterpret_cast<const float *>(ep.C) + (int64_t)m * ep.ldc + n;
        if (full && ep.c_vec) {
            const v4f c4 = *reinterpret_cast<const v4f *>(crow);
#pragma unroll
            for (int g = 0; g < 4; ++g)
                r[g] = fmaf(ep.beta, c4[g], r[g]);
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g)
                if (n + g < ep.N)
                    r[g] = fmaf(ep.beta, crow[g], r[g]);
        }
    } else if (ep.beta != 0.0f) {
        const uint16_t *crow = reinterpret_cast<const uint16_t *>(ep.C) + (int64_t)m * ep.ldc + n;
        if (full && ep.c_vec) {
            v2u c2 = *reinterpret_cast<const v2u *>(crow);
            r[0] = fmaf(ep.beta, bf16_to_f32(c2[0] & 0xFFFFu), r[0]);
            r[1] = fmaf(ep.beta, bf16_to_f32(c2[0] >> 16), r[1]);
            r[2] = fmaf(ep.beta, bf16_to_f32(c2[1] & 0xFFFFu), r[2]);
            r[3] = fmaf(ep.beta, bf16_to_f32(c2[1] >> 16), r[3]);
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g)
                if (n + g < ep.N)
                    r[g] = fmaf(ep.beta, bf16_to_f32(crow[g]), r[g]);
        }
    }
    uint16_t *drow = ep.D + (int64_t)m * ep.ldd + n;
    if (full && ep.d_vec) {
        v2u o;
        o[0] = bf16x2_rne(r[0], r[1]);
        o[1] = bf16x2_rne(r[2], r[3]);
        *reinterpret_cast<v2u *>(drow) = o;
    } else {
#pragma unroll
        for (int g = 0; g < 4; ++g)
            if (n + g < ep.N)
                drow[g] = (uint16_t)bf16_rne(r[g]);
    }
}

// bf16-atomic split-K: this chunk's alpha * acc, rounded to bf16, added into
// D with packed bf16 atomic adds (two columns per instruction).  Needs D
// 4-byte aligned and ldd, N even, so a pair never leaves its row; n is a
// multiple of 4.
__device__ __forceinline__ void atomic_add_quad(const Epilogue &ep, int m, int n, v4f acc)
{
    if (m >= ep.M || n >= ep.N)
        return;
    typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
    uint16_t *drow = ep.D + (int64_t)m * ep.ldd + n;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (n + 2 * h < ep.N) {
            const uint32_t w = bf16x2_rne(ep.alpha * acc[2 * h], ep.alpha * acc[2 * h + 1]);
            __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<v2bf_t *>(drow + 2 * h),
                                                       __builtin_bit_cast(v2bf_t, w));
        }
    }
}

// Map a hardware workgroup id to a logical one so that the workgroups the
// dispatcher sends to the same XCD (ids congruent mod 8) receive
// consecutive logical ids, i.e. neighbouring output tiles sharing operand
// rows in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int wg, int total)
{
    constexpr int kXcds = 8;
    const int xcd = wg % kXcds, idx = wg / kXcds;
    const int q = total / kXcds, r = total % kXcds;
    return xcd * q + (xcd < r ? xcd : r) + idx;
}

// ---- split-K partials shared between workgroups
//
// Workgroups of one output tile may run on different XCDs, whose L2 caches
// are not coherent with each other.  Partial sums are therefore written and
// read with the device-coherent cache policy (sc1, the policy the compiler
// uses for agent-scope atomic stores and loads): a store completes only once
// it is visible device-wide, and a load never hits a stale L2 line.  That
// makes the usual release/acquire fences, which write back and invalidate a
// whole L2 each time, unnecessary here.
constexpr int kCoherent = 16;  // cache-policy bits: sc1

__device__ __forceinline__ void store16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, v4f v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCoherent);
}

__device__ __forceinline__ v4f load16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent);
}

// Called by every thread after storing its part of the workgroup's partial
// with store16_coherent.  Returns true in exactly one workgroup of the tile
// (the last to arrive), whose threads may then read all partials with
// load16_coherent.  The counter is returned to zero for the next call.
// `flag`: an int in LDS that no thread accesses meanwhile.
__device__ __forceinline__ bool split_arrive_last_via(int *counter, int splits, int *flag)
{
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's partial stores are complete
    __syncthreads();                      // ... and so are every other thread's
    if (threadIdx.x == 0) {
        const int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = prev == splits - 1;
        if (last)
            __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last;
    }
    __syncthreads();
    return *flag != 0;
}

__device__ __forceinline__ bool split_arrive_last(int *counter, int splits)
{
    __shared__ int s_last;
    return split_arrive_last_via(counter, splits, &s_last);
}

}  // namespace mx

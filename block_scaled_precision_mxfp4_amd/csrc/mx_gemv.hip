// Single-row block-scaled GEMV (M == 1, row-major FP4 B; A in FP4, or FP8 /
// BF8 / FP6 below) on gfx950.
//
// The cost is reading B once from HBM.  A plain streaming read of B's bytes
// runs fastest in small pieces: many workgroups, each wave a few KiB.  This
// kernel gives a workgroup 4 rows of B (4 columns of D) and the whole of K;
// its four waves take 2048-K chunks of those rows in turn (chunk c to wave
// c mod 4), 4 KiB of B per chunk, and add their sums through LDS in wave
// order.  One chunk per wave at K = 8192.
//
// One scaled 16x16x128 FP4 instruction ("CDNA4 dense MFMA builtins",
// "Mixed-precision with scaling") covers 4 rows x 4 consecutive 128-K steps
// of B against all 16 steps of the chunk's A:
//   - B operand lane l (row x = l % 16 of the instruction's first operand,
//     K-block l / 16): B row x / 4, step 4t + x % 4 of the chunk for
//     instruction t = 0..3.  One load instruction then reads 256 contiguous
//     bytes of each of the 4 rows, and the four of a chunk the rows' whole
//     1 KiB.
//   - A operand lane l (column y = l % 16): step y of the chunk, K-block
//     l / 16 -- the chunk's 1 KiB of FP4 A in one load, the same for all
//     four instructions.
// Output (x, y) of instruction t is B row x / 4 at step 4t + x % 4 against A
// at step y; it is a term of the GEMV only where y = 4t + x % 4.  Lane l
// holds outputs x = 4 (l / 16) + i, y = l % 16 (i = 0..3), so its term is
// accumulator i = l % 4 of instruction t = (l % 16) / 4, for B row l / 16:
// each row's 16 terms sit in one 16-lane row of the wave.  The other outputs
// (an A step against a different B step) are never read.
//
// Scales follow their operand lanes: lane l's A scale is A's K-block
// (step l % 16, block l / 16); its B scale for instruction t is that of B
// row (l % 16) / 4, step 4t + l % 4, block l / 16.  Each lane loads one
// dword of scale bytes (A: step l % 16's four blocks; B: row l / 16, step
// l % 16) and the B words reach their operand lanes by a cross-lane permute;
// the lane's byte is shifted down for op_sel 0.
//
// AF: A's format (0 FP4; 1 FP8 E4M3, 2 BF8 E5M2, 3 FP6 E2M3, 4 FP6 E3M2;
// B is FP4).  A wider A operand lane holds its K-block as the skinny kernel
// does: 8-bit, the two 16-byte runs at bytes 16g and 64 + 16g of its step
// (g = l / 16); FP6, the block's 24 bytes.  A chunk of A is then 2 KiB or
// 1.5 KiB instead of 1 KiB; B and the scales are unchanged.
//
// MR (1 or 2): 2 <= M <= 4 * MR (FP4 A), the small-batch decode.  For each
// group of 4 A rows (one with MR = 1, two with MR = 2, sharing every B
// operand and B scale word, with an accumulator each) the A operand's lanes
// then pair like B's: lane y = l % 16 carries A row y / 4 at step 4t + y % 4
// (one 16-byte load per lane and instruction: 256 contiguous bytes of each
// of the 4 rows, rows past M loading nothing), and its scale words reach
// their lanes by the same permute as B's.  Output (x, y) is a term where the
// two steps agree, x % 4 = y % 4, for B row x / 4 and A row y / 4; those
// positions are the same in every instruction, so one accumulator sums the
// chunk: lane l's term is element l % 4, for A row (l % 16) / 4 and B row
// l / 16, and each (A row, B row) pair's four terms sit in one lane quad.
//
// Requires K % 2048 == 0 (every chunk whole: no range checks inside K, no
// scale bytes of a neighbouring row), 16-byte aligned scale rows, split 1.
#include "mx_args.hpp"
#include "mx_device.hpp"

#include <type_traits>

namespace mx {

constexpr int kGemvRows = 4;     // rows of B (columns of D) per workgroup
constexpr int kGemvChunk = 2048; // K per chunk: 16 steps of 128

template <int AF, int MR>
struct GemvChunk {
    using a_t = typename std::conditional<AF == 0, v4i, v8i>::type;
    v4i b[4];     // B operand of instruction t
    a_t a;        // A operand, all 16 steps of the chunk (one row)
    v4i am[MR ? 4 * MR : 1];  // MR: A operand of instruction t, row group h: am[4h + t]
    uint32_t sa;  // A scale bytes of step l % 16 (MR: of row l / 16)
    uint32_t sa_hi;  // MR = 2: of row 4 + l / 16
    uint32_t sb;  // B scale bytes of row l / 16, step l % 16
};

// Loads of chunk c (nothing, without memory traffic, when !on).  The scale
// words and the A operand go first: the scale permutes can then start while
// B is still arriving, and each multiply waits only for its own B operand.
template <int AF, int MR>
__device__ __forceinline__ void gemv_issue(GemvChunk<AF, MR> &ch, int c, bool on, __amdgpu_buffer_rsrc_t rb,
                                           __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rsa,
                                           __amdgpu_buffer_rsrc_t rsb, uint32_t b_lane, uint32_t sb_lane,
                                           const uint32_t (&a_lane)[2], const uint32_t (&sa_lane)[2], int lane)
{
    const uint32_t bc = (uint32_t)c * (kGemvChunk / 2);
    ch.sb = load4(rsb, on && sb_lane != kOOB ? sb_lane + (uint32_t)c * 64 : kOOB);
    if constexpr (MR > 0) {
        ch.sa = load4(rsa, on && sa_lane[0] != kOOB ? sa_lane[0] + (uint32_t)c * 64 : kOOB);
        if constexpr (MR > 1)
            ch.sa_hi = load4(rsa, on && sa_lane[1] != kOOB ? sa_lane[1] + (uint32_t)c * 64 : kOOB);
#pragma unroll
        for (int h = 0; h < MR; ++h)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                ch.am[4 * h + t] = load16(ra, on && a_lane[h] != kOOB ? a_lane[h] + bc + t * 256 : kOOB);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            ch.b[t] = load16_stream(rb, on && b_lane != kOOB ? b_lane + bc + t * 256 : kOOB);
        return;
    }
    ch.sa = load4(rsa, on ? (uint32_t)c * 64 + (lane & 15) * 4 : kOOB);
    constexpr int AKB = 4 * kFmtBits[AF];  // bytes of an A K-block
    const uint32_t ac = (uint32_t)c * 64 * AKB + (lane & 15) * 4 * AKB;  // the lane's step
    if constexpr (AF == 0) {
        ch.a = load16(ra, on ? ac + (lane >> 4) * 16 : kOOB);
    } else if constexpr (kFmtBits[AF] == 8) {
        const uint32_t o = ac + (lane >> 4) * 16;
        const v4i lo = load16(ra, on ? o : kOOB), hi = load16(ra, on ? o + 64 : kOOB);
        ch.a = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
        const uint32_t o = ac + (lane >> 4) * 24;
        const v4i lo = load16(ra, on ? o : kOOB);
        const v2u hi = load8(ra, on ? o + 16 : kOOB);
        ch.a = v8i{lo[0], lo[1], lo[2], lo[3], (int)hi[0], (int)hi[1], 0, 0};
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
        ch.b[t] = load16_stream(rb, on && b_lane != kOOB ? b_lane + bc + t * 256 : kOOB);
}

template <int AF, int MR>
__device__ __forceinline__ void gemv_compute(const GemvChunk<AF, MR> &ch, v4f (&acc)[4], int lane)
{
    const int sh = 8 * (lane >> 4);
    const int q = lane & 15;
    if constexpr (MR > 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            // B's and A's scale words of this lane: row q / 4 of each (of the
            // A row group), step 4t + q % 4 of the chunk
            const int src = (q >> 2) * 16 + 4 * t + (q & 3);
            const uint32_t wb = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)ch.sb);
#pragma unroll
            for (int h = 0; h < MR; ++h) {
                const uint32_t wa = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)(h ? ch.sa_hi : ch.sa));
                acc[h] = mfma_fp4<0, 0>(ch.b[t], ch.am[4 * h + t], acc[h], (int)(wb >> sh), (int)(wa >> sh));
            }
        }
        return;
    }
    const int sa = (int)(ch.sa >> sh);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        // this lane's B scale word: row q / 4, step 4t + q % 4 of the chunk
        const int src = (q >> 2) * 16 + 4 * t + (q & 3);
        const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)ch.sb);
        if constexpr (AF == 0)
            acc[t] = mfma_fp4<0, 0>(ch.b[t], ch.a, acc[t], (int)(w >> sh), sa);
        else
            acc[t] = mfma_fp4_wide<kFmtHw[AF], 0, 0>(ch.b[t], ch.a, acc[t], (int)(w >> sh), sa);
    }
}

// LOOP = false: at most one chunk per wave (K <= 8192), one register set.
template <int AF, bool LOOP, int MR>
__device__ __forceinline__ void gemv_body(const GemmArgs &g)
{
    __shared__ float s_part[4][MR ? 4 * MR : 1][kGemvRows];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * kGemvRows;
    const int rows = min(kGemvRows, g.N - n0);
    const uint32_t kbytes = (uint32_t)(g.K / 2);
    const auto rb = make_rsrc(g.B + (int64_t)n0 * g.ldb_b, (uint32_t)((rows - 1) * g.ldb_b) + kbytes);
    const auto rsb = make_rsrc(g.SB + (int64_t)n0 * g.ldsb, (uint32_t)((rows - 1) * g.ldsb + g.KB));
    const auto ra = make_rsrc(g.A, (uint32_t)((int64_t)(MR ? g.M - 1 : 0) * g.lda_b + (int64_t)g.K * kFmtBits[AF] / 8));
    const auto rsa = make_rsrc(g.SA, (uint32_t)((int64_t)(MR ? g.M - 1 : 0) * g.ldsa + g.KB));
    static_assert(MR <= 2, "at most two groups of 4 A rows");

    // per-lane offsets inside a chunk: B row (l % 16) / 4 at step l % 4 of
    // the instruction's four, K-block l / 16; B scale dword: row l / 16,
    // step l % 16.  Rows past N load nothing.
    const int br = (lane & 15) >> 2;
    const uint32_t b_lane = br < rows ? (uint32_t)(br * g.ldb_b) + (lane & 3) * 64 + (lane >> 4) * 16 : kOOB;
    const int sr = lane >> 4;
    const uint32_t sb_lane = sr < rows ? (uint32_t)(sr * g.ldsb) + (lane & 15) * 4 : kOOB;
    // MR: A row 4h + (l % 16) / 4 as B's, and its scale dword row 4h + l / 16
    uint32_t a_lane[2], sa_lane[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int ar = 4 * h + br, asr = 4 * h + sr;
        a_lane[h] = MR > h && ar < g.M ? (uint32_t)(ar * g.lda_b) + (lane & 3) * 64 + (lane >> 4) * 16 : kOOB;
        sa_lane[h] = MR > h && asr < g.M ? (uint32_t)(asr * g.ldsa) + (lane & 15) * 4 : kOOB;
    }

    v4f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

    const int chunks = g.K / kGemvChunk;
    int c = wave;
    if (c < chunks) {
        GemvChunk<AF, MR> x;
        gemv_issue(x, c, true, rb, ra, rsa, rsb, b_lane, sb_lane, a_lane, sa_lane, lane);
        if (!LOOP) {
            gemv_compute(x, acc, lane);
        } else if (c + 4 >= chunks) {
            gemv_compute(x, acc, lane);  // one chunk for this wave (K <= 8192)
        } else {
            // two register sets: each chunk's loads are issued before the
            // previous chunk's multiplies.  Every pass issues and multiplies
            // both sets (a chunk past K loads nothing and adds zeros), so no
            // load is conditional and each multiply waits only for its own
            // operands.
            GemvChunk<AF, MR> y;
            const int mine = (chunks - wave + 3) / 4;  // this wave's chunks
            for (int i = 0; i < mine; i += 2) {
                gemv_issue(y, c + 4, c + 4 < chunks, rb, ra, rsa, rsb, b_lane, sb_lane, a_lane, sa_lane, lane);
                gemv_compute(x, acc, lane);
                gemv_issue(x, c + 8, c + 8 < chunks, rb, ra, rsa, rsb, b_lane, sb_lane, a_lane, sa_lane, lane);
                gemv_compute(y, acc, lane);
                c += 8;
            }
        }
    }

    if constexpr (MR > 0) {
        // the lane's term of row group h: element l % 4 of accumulator h,
        // for A row 4h + (l % 16) / 4 and B row l / 16; a quad (lane ^ 1,
        // lane ^ 2) holds one pair's four terms
        const int ii = lane & 3;
#pragma unroll
        for (int h = 0; h < MR; ++h) {
            float v = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i == ii)
                    v = acc[h][i];
            v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
            v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
            if ((lane & 3) == 0)
                s_part[wave][4 * h + ((lane & 15) >> 2)][lane >> 4] = v;
        }
        __syncthreads();
        if (threadIdx.x < g.M) {
            const int m = threadIdx.x;
            v4f tot;
#pragma unroll
            for (int r = 0; r < kGemvRows; ++r) {
                float s = s_part[0][m][r];
#pragma unroll
                for (int w = 1; w < 4; ++w)
                    s += s_part[w][m][r];
                tot[r] = s;
            }
            Epilogue ep{g.D, g.C, g.alpha, g.beta, g.M, g.N, g.ldd, g.ldc, g.d_vec, g.c_vec, g.c_f32};
            store_quad(ep, m, n0, tot);
        }
        return;
    }
    // the lane's term: accumulator l % 4 of instruction (l % 16) / 4
    const int ti = (lane & 15) >> 2, ii = lane & 3;
    float v = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (t == ti && i == ii)
                v = acc[t][i];
    // sum of the 16 lanes of each row: quad (lane ^ 1, lane ^ 2), then the
    // mirrored half-row and row partners, so every lane ends with its row's
    // total in one fixed order
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
    if ((lane & 15) == 0)
        s_part[wave][0][lane >> 4] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        v4f tot;
#pragma unroll
        for (int r = 0; r < kGemvRows; ++r) {
            float s = s_part[0][0][r];
#pragma unroll
            for (int w = 1; w < 4; ++w)
                s += s_part[w][0][r];
            tot[r] = s;
        }
        Epilogue ep{g.D, g.C, g.alpha, g.beta, g.M, g.N, g.ldd, g.ldc, g.d_vec, g.c_vec, g.c_f32};
        store_quad(ep, 0, n0, tot);
    }
}

template <int AF, int MR>
__global__ void __launch_bounds__(256) mx_gemv_kernel(GemmArgs g)
{
    gemv_body<AF, true, MR>(g);
}

// One chunk per wave: at most 64 registers, so that eight waves fit a SIMD
// and all 2048 workgroups of N = 8192 are resident at once.
template <int AF, int MR>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) mx_gemv1_kernel(GemmArgs g)
{
    gemv_body<AF, false, MR>(g);
}

template <int AF, int MR>
static void launch_gemv_fmt(const GemmArgs &g, int grid, hipStream_t s)
{
    if (g.K <= 4 * kGemvChunk)
        hipLaunchKernelGGL((mx_gemv1_kernel<AF, MR>), dim3(grid), dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL((mx_gemv_kernel<AF, MR>), dim3(grid), dim3(256), 0, s, g);
}

void launch_gemv(int a_fmt, const GemmArgs &g, int grid, hipStream_t s)
{
    if (g.M > 4) {  // 5 <= M <= 8, FP4 A
        launch_gemv_fmt<0, 2>(g, grid, s);
        return;
    }
    if (g.M > 1) {  // 2 <= M <= 4, FP4 A
        launch_gemv_fmt<0, 1>(g, grid, s);
        return;
    }
    switch (a_fmt) {
    case 0: launch_gemv_fmt<0, 0>(g, grid, s); break;
    case 1: launch_gemv_fmt<1, 0>(g, grid, s); break;
    case 2: launch_gemv_fmt<2, 0>(g, grid, s); break;
    case 3: launch_gemv_fmt<3, 0>(g, grid, s); break;
    default: launch_gemv_fmt<4, 0>(g, grid, s); break;
    }
}

}  // namespace mx

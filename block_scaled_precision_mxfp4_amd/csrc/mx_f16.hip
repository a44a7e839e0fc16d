// FP16 GEMM with transposed LDS reads on gfx950 -- the FP16 example of
// "CDNA4 MFMA transpose load builtins" ("FP16 GEMM example"), rebuilt around
// the same staging as the MXFP4 tiled kernel.
//
//     C[M,N] (fp32) = A[M,K] (fp16, row-major) x B[K,N] (fp16, row-major)
//
// B is stored K-major in memory (row k holds N consecutive columns), so a
// lane's B operand -- one column, 8 consecutive K -- is strided in memory.
// Both tiles move HBM/L2 -> LDS unchanged with 16-byte direct-to-LDS loads;
// A fragments are plain 16-byte LDS reads (row lane%16, K 8g..8g+7 with
// g = lane/16), and B fragments come from two ds_read_b64_tr_b16 per
// 32-K step: 16 lanes name 4 K-rows x 16 columns and each receives its own
// column's 4 K values (the page's "Step 2", calls 1 and 2 four K-rows
// apart).  One v_mfma_f32_16x16x32_f16 consumes the 8 K of 16 rows x 16
// columns per lane group.
//
// Block 256 x 256, eight waves of 128 x 64 (two per SIMD), 64-K stages,
// double-buffered (128 KiB of LDS):
//   A stage: 256 rows x 128 bytes; a load instruction covers 8 whole rows,
//            16-byte chunk c of row r stored at slot c ^ ((r/2) % 8), so the
//            16 rows of a fragment read hit 16 different bank groups;
//   B stage: 64 K-rows x 512 bytes; a load covers 2 K-rows, chunk c of
//            K-row k stored at slot c ^ h(k), h(k) = 2 * ((k % 4) + 4 *
//            ((k / 8) % 2)): the 8 K-rows a half-wave of transposed reads
//            touches (each a 32-byte run of one column block) land on 8
//            different 32-byte bank ranges.
// Edges: rows past M read zeros through the buffer range; K and N are
// whole 16-byte chunks (K % 8 == 0, N % 8 == 0) and chunks past them load
// zeros; stores are masked.
#include "mx_args.hpp"
#include "mx_device.hpp"

#include <type_traits>

namespace mx {

typedef __fp16 v4h_t __attribute__((ext_vector_type(4)));
typedef _Float16 v8f16_t __attribute__((ext_vector_type(8)));

// all vector-memory operations of this wave done (loads into LDS included)
__device__ __forceinline__ void f16_wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ v4h_t lds_tr16(const uint8_t *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4f16(
        (__attribute__((address_space(3))) v4h_t *)(reinterpret_cast<const __fp16 *>(p)));
}

__global__ void __launch_bounds__(512) mx_f16_kernel(F16Args g)
{
    constexpr int BM = 256, BN = 256, BK = 64;
    constexpr int WM = 2, WN = 4;           // waves
    constexpr int TM = BM / WM, TN = BN / WN;  // 128 x 64 per wave
    constexpr int FM = TM / 16, FN = TN / 16;  // 8 x 4 fragments
    constexpr int A_ROW = BK * 2;              // 128 bytes of a row per stage
    constexpr int B_ROW = BN * 2;              // 512 bytes of a K-row per stage
    constexpr int A_STAGE = BM * A_ROW, B_STAGE = BK * B_ROW;  // 32 KiB each
    constexpr int A_LD = A_STAGE / 1024 / 8, B_LD = B_STAGE / 1024 / 8;  // loads per wave
    __shared__ __attribute__((aligned(1024))) uint8_t s_a0[A_STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t s_a1[A_STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t s_b0[B_STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t s_b1[B_STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave % WM, wave_n = wave / WM;

    // tile order: groups of 4 tile rows, column-major inside a group
    const int lg = xcd_remap(blockIdx.x, gridDim.x);
    const int per_group = 4 * g.tiles_n;
    const int grp = lg / per_group, first_m = grp * 4;
    const int gsz = min(g.tiles_m - first_m, 4);
    const int within = lg - grp * per_group;
    const int m0 = (first_m + within % gsz) * BM, n0 = (within / gsz) * BN;
    const int nst = (g.K + BK - 1) / BK;

    const int rows_a = min(BM, g.M - m0);
    const auto ra = make_rsrc(g.A + (int64_t)m0 * g.lda_b, (uint32_t)(rows_a * g.lda_b));
    const auto rb = make_rsrc_u(g.B, (uint32_t)((int64_t)g.K * g.ldb_b));  // the host keeps it below 2^31

    // per-lane parts of the load addresses: A lane s of an instruction
    // fills row s/8, slot s%8; B lane s fills K-row s/32, slot s%32
    const int a_r = lane >> 3, a_slot = lane & 7;
    const int b_k = lane >> 5, b_slot = lane & 31;

    auto issue = [&](int kt, auto bufc) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        uint8_t *da = BUF ? s_a1 : s_a0;
        uint8_t *db = BUF ? s_b1 : s_b0;
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int q = i * 8 + wave;  // instruction: rows 8q .. 8q+7
            const int r = q * 8 + a_r;
            const int c = a_slot ^ ((r >> 1) & 7);  // the chunk this slot holds
            const int k = k0 + c * 8;
            load16_to_lds(ra, (lds_void *)(da + q * 1024),
                          k < g.K ? (uint32_t)(r * g.lda_b + k * 2) : kOOB);
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int q = i * 8 + wave;  // instruction: K-rows 2q, 2q+1
            const int kr = q * 2 + b_k;
            const int h = 2 * ((kr & 3) + 4 * ((kr >> 3) & 1));
            const int c = b_slot ^ h;
            const int k = k0 + kr, n = n0 + c * 8;
            load16_to_lds(rb, (lds_void *)(db + q * 1024),
                          k < g.K && n < g.N ? (uint32_t)(k * g.ldb_b + n * 2) : kOOB);
        }
    };

    // fragment reads
    const int fr = lane & 15, fg = lane >> 4;
    // A: row wave_m*TM + fm*16 + fr, chunk ks*4 + fg
    auto a_addr = [&](int fm, int ks) __attribute__((always_inline)) {
        const int r = wave_m * TM + fm * 16 + fr;
        return r * A_ROW + (((ks * 4 + fg) ^ ((r >> 1) & 7)) * 16);
    };
    // B (call 0/1): K-row ks*32 + 8*fg + 4*call + fr/4, columns
    // wave_n*TN + fn*16 + 4*(fr%4) .. +3 (8 bytes)
    auto b_addr = [&](int fn, int ks, int call) __attribute__((always_inline)) {
        const int kr = ks * 32 + 8 * fg + 4 * call + (fr >> 2);
        const int col = wave_n * TN + fn * 16 + 4 * (fr & 3);
        const int c = col >> 3, half = (col >> 2) & 1;
        const int h = 2 * ((kr & 3) + 4 * ((kr >> 3) & 1));
        return kr * B_ROW + ((c ^ h) * 16) + half * 8;
    };

    v4f acc[FN][FM];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            acc[fn][fm] = v4f{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](auto bufc) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        const uint8_t *sa = BUF ? s_a1 : s_a0;
        const uint8_t *sb = BUF ? s_b1 : s_b0;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            v8f16_t af[FM];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                af[fm] = *reinterpret_cast<const v8f16_t *>(sa + a_addr(fm, ks));
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const v4h_t lo = lds_tr16(sb + b_addr(fn, ks, 0));
                const v4h_t hi = lds_tr16(sb + b_addr(fn, ks, 1));
                const v8f16_t bf = {(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
                                    (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]};
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fn][fm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[fm], bf, acc[fn][fm], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    auto stage = [&](int kt, auto bufc) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        if (kt + 1 < nst)
            issue(kt + 1, std::integral_constant<int, BUF ^ 1>{});
        compute(bufc);
        f16_wait_vmem();
        __syncthreads();
    };

    issue(0, B0{});
    f16_wait_vmem();
    __syncthreads();
    int kt = 0;
    for (; kt + 2 <= nst; kt += 2) {
        stage(kt, B0{});
        stage(kt + 1, B1{});
    }
    if (kt < nst)
        stage(kt, B0{});

    // epilogue: lane holds rows 4*fg + i of each 16 x 16 block, column fr
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int n = n0 + wave_n * TN + fn * 16 + fr;
        if (n >= g.N)
            continue;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + wave_m * TM + fm * 16 + 4 * fg + i;
                if (m < g.M)  // C is written once: the non-temporal hint (3 % faster at 8192^3)
                    __builtin_nontemporal_store(acc[fn][fm][i], &g.C[(int64_t)m * g.ldc + n]);
            }
    }
}

int64_t f16_grid(int M, int N) { return (int64_t)((M + 255) / 256) * ((N + 255) / 256); }

void launch_f16(const F16Args &a, int64_t grid, hipStream_t s)
{
    hipLaunchKernelGGL(mx_f16_kernel, dim3((unsigned)grid), dim3(512), 0, s, a);
}

}  // namespace mx

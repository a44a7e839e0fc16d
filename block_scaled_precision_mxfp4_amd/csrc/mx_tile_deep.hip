// Deep-pipelined tiled MXFP4 GEMM for gfx950 (the main dense kernel).
//
// Same tile shape, fragment layout and epilogue as mx_tile_kernel, with a
// longer software pipeline: each 128-K step of the tile is one stage, and a
// ring of NS = 4 LDS stage buffers lets the loads of step kt+3 be in flight
// while step kt is multiplied (about 3000 matrix-unit cycles of latency
// cover at the 256x256 tile, against ~1000 for a two-buffer ring).
//
// Every byte a stage needs moves HBM/L2 -> LDS with direct-to-LDS buffer
// loads, scales included: row-major scale rows contribute one 4-byte word
// (the row's 4 K-blocks of the step) per row, packed B scales one 256-byte
// chunk per 32-row group.  Each wave issues the same number of loads per
// stage (idle slots load from an empty range), so "stage kt has landed" is
// an exact s_waitcnt on the number of loads issued after it, followed by one
// workgroup barrier; that barrier also frees the buffer of step kt-1 for the
// loads of step kt+3.
//
// Requirements (checked by the host, otherwise mx_tile_kernel runs): scale
// rows 4-byte aligned, K a multiple of 128.
#include "mx_args.hpp"
#include "mx_device.hpp"
#include "mx_pipe.hpp"

#include <type_traits>

namespace mx {


template <int BM, int BN, int WM, int WN, bool BPACK, bool SAPACK>
__global__ void __launch_bounds__(64 * WM * WN) mx_tile_deep_kernel(GemmArgs g)
{
    constexpr int NS = 4;                      // stage buffers
    constexpr int NW = WM * WN;                // waves
    constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
    constexpr int FM = TM / 16, FN = TN / 16;  // 16-row fragments per wave
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    static_assert(FN % 2 == 0, "packed scale words cover 32-row groups");
    constexpr int A_CH = BM / 16, B_CH = BN / 16;  // 1 KiB operand chunks per stage
    static_assert(A_CH % NW == 0 && B_CH % NW == 0, "chunks split evenly over waves");
    constexpr int A_STAGE = BM * 64, B_STAGE = BN * 64;  // operand bytes per stage
    // scale loads per stage (64 lanes x 4 bytes each)
    constexpr int SA_I = SAPACK ? BM / 32 : BM / 64;  // row-major A: one word per row
    constexpr int SB_I = BPACK ? BN / 32 : BN / 64;   // packed: one 256-byte chunk per 32 rows
    static_assert(BM % 64 == 0 && (BPACK ? BN % 32 == 0 : BN % 64 == 0), "whole scale loads");
    constexpr int SC_I = SA_I + SB_I;
    constexpr int SC_PER_WAVE = (SC_I + NW - 1) / NW;
    constexpr int SA_BYTES = SAPACK ? BM / 32 * 256 : BM * 4, SB_BYTES = BPACK ? BN / 32 * 256 : BN * 4;
    constexpr int L = A_CH / NW + B_CH / NW + SC_PER_WAVE;  // loads per wave per stage
    static_assert((NS - 2) * L < 64, "vmcnt range");

    // One LDS block; regions at compile-time offsets: [A slots][B slots]
    // [A scale slots][B scale slots][idle row].  Fragment reads are asm with immediate
    // offsets from one base register per region.
    constexpr int OFF_B = NS * A_STAGE;
    constexpr int OFF_SA = OFF_B + NS * B_STAGE;
    constexpr int OFF_SB = OFF_SA + NS * SA_BYTES;
    // idle load slots still write (zeros) to LDS: they get a row nobody reads
    constexpr int OFF_IDLE = OFF_SB + NS * SB_BYTES;
    constexpr int LDS_BYTES = OFF_IDLE + 256;
    static_assert(A_STAGE <= 65536 && B_STAGE <= 65536, "a slot fits the ds offset field");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave % WM, wave_n = wave / WM;

    // ---- which tile and K chunk (as in mx_tile_kernel)
    const int tiles = g.tiles_m * g.tiles_n;
    const int lg = xcd_remap(blockIdx.x, gridDim.x);
    const int z = lg / tiles;
    const int t = lg - z * tiles;
    const int per_group = g.group_m * g.tiles_n;
    const int grp = t / per_group;
    const int first_m = grp * g.group_m;
    const int gsz = min(g.tiles_m - first_m, g.group_m);
    const int within = t - grp * per_group;
    const int tm = first_m + within % gsz;
    const int tn = within / gsz;
    const int m0 = tm * BM, n0 = tn * BN;

    const int kb_begin = z * g.kb_per_split;
    const int kb_end = min(g.KB, kb_begin + g.kb_per_split);
    const int nst = (kb_end - kb_begin) >> 2;  // 128-K steps (K is a multiple of 128)

    // ---- sources, rebased at the tile; a stage moves the base along K
    const int rows_a = min(BM, g.M - m0);
    const uint8_t *a_base = g.A + (int64_t)m0 * g.lda_b;
    const uint32_t a_bytes = (uint32_t)(rows_a * g.lda_b);
    const uint32_t a_lane = (uint32_t)((lane & 15) * g.lda_b + (lane >> 4) * 16);
    const uint8_t *sa_base;
    uint32_t sa_bytes;
    if constexpr (SAPACK) {
        const int m32 = m0 / 32, grp32 = min(BM / 32, (g.M + 31) / 32 - m32);
        sa_base = g.SA + (int64_t)m32 * g.sn8 * 256;
        sa_bytes = (uint32_t)(grp32 * g.sn8 * 256);
    } else {
        sa_base = g.SA + (int64_t)m0 * g.ldsa;
        sa_bytes = (uint32_t)(rows_a * g.ldsa);
    }
    const uint8_t *b_base, *sb_base;
    uint32_t b_bytes, b_lane, b_rg_stride, sb_bytes;
    if constexpr (BPACK) {
        const int n16 = n0 / 16, grp16 = min(BN / 16, (g.N + 15) / 16 - n16);
        b_base = g.B + (int64_t)n16 * g.ks_total * 1024;
        b_bytes = (uint32_t)(grp16 * g.ks_total * 1024);
        b_lane = (uint32_t)(lane * 16);
        b_rg_stride = (uint32_t)(g.ks_total * 1024);
        const int n32 = n0 / 32, grp32 = min(BN / 32, (g.N + 31) / 32 - n32);
        sb_base = g.SB + (int64_t)n32 * g.sn8 * 256;
        sb_bytes = (uint32_t)(grp32 * g.sn8 * 256);
    } else {
        const int rows_b = min(BN, g.N - n0);
        b_base = g.B + (int64_t)n0 * g.ldb_b;
        b_bytes = (uint32_t)(rows_b * g.ldb_b);
        b_lane = (uint32_t)((lane & 15) * g.ldb_b + (lane >> 4) * 16);
        b_rg_stride = (uint32_t)(16 * g.ldb_b);
        sb_base = g.SB + (int64_t)n0 * g.ldsb;
        sb_bytes = (uint32_t)(rows_b * g.ldsb);
    }

    // ---- one stage's loads (exactly L per wave; `on` false: empty ranges)
    auto issue = [&](int kt, bool on, int slot) {
        uint8_t *sa_ = smem + slot * A_STAGE, *sb_ = smem + OFF_B + slot * B_STAGE;
        uint8_t *ssa = smem + OFF_SA + slot * SA_BYTES, *ssb = smem + OFF_SB + slot * SB_BYTES;
        const int kb_s = kb_begin + kt * 4;
        const uint32_t a_k = (uint32_t)kb_s * 16;
        const uint32_t b_k = BPACK ? (uint32_t)(kb_s >> 2) * 1024 : (uint32_t)kb_s * 16;
        const auto ra = make_rsrc(a_base + a_k, on ? a_bytes - a_k : 0u);
        const auto rb = make_rsrc(b_base + b_k, on ? b_bytes - b_k : 0u);
#pragma unroll
        for (int i = 0; i < A_CH / NW; ++i) {
            const int rg = i * NW + wave;
            load16_to_lds(ra, (lds_void *)(sa_ + rg * 1024), a_lane + (uint32_t)(rg * 16 * g.lda_b));
        }
#pragma unroll
        for (int i = 0; i < B_CH / NW; ++i) {
            const int rg = i * NW + wave;
            load16_to_lds(rb, (lds_void *)(sb_ + rg * 1024), b_lane + (uint32_t)rg * b_rg_stride);
        }
        // scale loads, round-robin over the waves; slots past SC_I are idle
        const uint32_t sa_k = SAPACK ? (uint32_t)(kb_s >> 3) * 256 : (uint32_t)kb_s;
        const auto rsa = make_rsrc(sa_base + sa_k, on ? sa_bytes - sa_k : 0u);
        uint32_t sb_k;
        if constexpr (BPACK)
            sb_k = (uint32_t)(kb_s >> 3) * 256;  // 8-block group of this step
        else
            sb_k = (uint32_t)kb_s;
        const auto rsb = make_rsrc(sb_base + sb_k, on ? sb_bytes - sb_k : 0u);
#pragma unroll
        for (int i = 0; i < SC_PER_WAVE; ++i) {
            const int c = i * NW + wave;  // wave-uniform
            if (c < SA_I) {
                const int row = c * 64 + lane;
                const uint32_t off = SAPACK ? (uint32_t)((c * g.sn8 * 64 + lane) * 4) : (uint32_t)(row * g.ldsa);
                load4_to_lds(rsa, (lds_void *)(ssa + c * 256), off);
            } else if (c < SC_I) {
                const int cb = c - SA_I;
                uint32_t off;
                if constexpr (BPACK)
                    off = (uint32_t)((cb * g.sn8 * 64 + lane) * 4);
                else
                    off = (uint32_t)((cb * 64 + lane) * g.ldsb);
                load4_to_lds(rsb, (lds_void *)(ssb + cb * 256), off);
            } else {
                // keep the per-stage load count uniform across waves; an
                // out-of-range direct load still writes zeros to its LDS row
                load4_to_lds(rsb, (lds_void *)(smem + OFF_IDLE), kOOB);
            }
        }
    };

    // ---- fragment read bases (one register per LDS region; ring slot and
    // fragment offsets are instruction immediates)
    const uint32_t lds0 = lds_addr(smem);
    const uint32_t base_a = lds0 + (uint32_t)(wave_m * FM * 1024 + lane * 16);
    const uint32_t base_b = lds0 + (uint32_t)(OFF_B + wave_n * FN * 1024 + lane * 16);
    const uint32_t base_sa =
        SAPACK ? lds0 + (uint32_t)(OFF_SA + wave_m * (TM / 32) * 256 + lane * 4)
               : lds0 + (uint32_t)(OFF_SA + (wave_m * TM + (lane & 15)) * 4 + (lane >> 4));
    uint32_t base_sb;
    if constexpr (BPACK)
        base_sb = lds0 + (uint32_t)(OFF_SB + wave_n * (TN / 32) * 256 + lane * 4);
    else
        base_sb = lds0 + (uint32_t)(OFF_SB + (wave_n * TN + (lane & 15)) * 4 + (lane >> 4));

    // ---- accumulators: first defined by the first stage's instructions
    v4f acc[FN][FM];

    auto compute = [&](int kt, auto firstc) {
        constexpr bool FIRST = decltype(firstc)::value;
        const int slot = kt & (NS - 1);
        const uint32_t ra_ = base_a + slot * A_STAGE, rb_ = base_b + slot * B_STAGE;
        const uint32_t rsa_ = base_sa + slot * SA_BYTES, rsb_ = base_sb + slot * SB_BYTES;
        // scales: row-major words hold the row's 4 blocks of this step, the
        // lane takes byte lane/16 (op_sel 0); packed words hold two steps x
        // two row halves: shifted so that this step's halves are bytes 0, 1
        // (chunks start on even steps, so the step parity is kt's)
        constexpr int NSB = BPACK ? FN / 2 : FN;
        constexpr int NSA = SAPACK ? FM / 2 : FM;
        uint32_t sav[NSA], sbv[NSB];
        v4i af[FM], bfr[FN];
        if constexpr (SAPACK) {
            static_for<FM / 2>([&](auto i) {
                constexpr int p = decltype(i)::value;
                sav[p] = lds_read4<p * 256>(rsa_);
            });
        } else {
            static_for<FM>([&](auto i) {
                constexpr int fm = decltype(i)::value;
                sav[fm] = lds_read1<fm * 64>(rsa_);
            });
        }
        if constexpr (BPACK) {
            static_for<FN / 2>([&](auto i) {
                constexpr int p = decltype(i)::value;
                sbv[p] = lds_read4<p * 256>(rsb_);
            });
        } else {
            static_for<FN>([&](auto i) {
                constexpr int fn = decltype(i)::value;
                sbv[fn] = lds_read1<fn * 64>(rsb_);
            });
        }
        static_for<FN>([&](auto i) {
            constexpr int fn = decltype(i)::value;
            bfr[fn] = lds_read16<fn * 1024>(rb_);
        });
        static_for<FM>([&](auto i) {
            constexpr int fm = decltype(i)::value;
            af[fm] = lds_read16<fm * 1024>(ra_);
        });
        // scales and B fragments first; then one column of multiplies per A
        // fragment as soon as that fragment has landed
        lds_wait_n<FM>(sav, sbv, bfr);
        if constexpr (BPACK) {
            const int sh = (kt & 1) * 16;
#pragma unroll
            for (int p = 0; p < FN / 2; ++p)
                sbv[p] >>= sh;
        }
        if constexpr (SAPACK) {
            const int sh = (kt & 1) * 16;
#pragma unroll
            for (int p = 0; p < FM / 2; ++p)
                sav[p] >>= sh;
        }
        static_for<FM>([&](auto i) {
            constexpr int fm = decltype(i)::value;
            lds_wait_n<FM - 1 - fm>(af[fm]);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int ob = BPACK ? (fn & 1) : 0;
                constexpr int oa = SAPACK ? (fm & 1) : 0;
                acc[fn][fm] = mma_sel(ob, oa, bfr[fn], af[fm], FIRST ? v4f{0.f, 0.f, 0.f, 0.f} : acc[fn][fm],
                                      (int)sbv[BPACK ? fn / 2 : fn], (int)sav[SAPACK ? fm / 2 : fm]);
            }
        });
    };

    using First = std::true_type;
    using Rest = std::false_type;
    // stage kt: wait for its loads (the NS-2 later stages may stay in flight),
    // barrier, refill the slot freed by step kt-1 with step kt+NS-1, multiply.
    // One stage per loop iteration keeps register pressure at one stage's
    // fragments; the ring slot is a runtime value (uniform, scalar).
    auto stage = [&](int kt, auto firstc) {
        __builtin_amdgcn_sched_barrier(0);
        stage_sync<(NS - 2) * L>();
        issue(kt + NS - 1, kt + NS - 1 < nst, (kt + NS - 1) & (NS - 1));
        compute(kt, firstc);
        __builtin_amdgcn_sched_barrier(0);  // this stage's multiplies stay in this stage
    };

    issue(0, true, 0);
    issue(1, 1 < nst, 1);
    issue(2, 2 < nst, 2);
    stage(0, First{});
    for (int kt = 1; kt < nst; ++kt)
        stage(kt, Rest{});
    wait_vmcnt<0>();  // idle loads of the last stages

    // ---- epilogue (as in mx_tile_kernel)
    Epilogue ep{g.D, g.C, g.alpha, g.beta, g.M, g.N, g.ldd, g.ldc, g.d_vec, g.c_vec, g.c_f32};
    const int mb = m0 + wave_m * TM + (lane & 15);
    const int nb = n0 + wave_n * TN + 4 * (lane >> 4);
    if (g.split == 1) {
        if (g.d_stage) {
            // all waves' loads (idle ones included) have landed and all
            // fragment reads are done: the ring is free for the staging
            __syncthreads();
            constexpr int REG = TM * TN * 2;
            static_assert(NW * REG <= LDS_BYTES, "staging regions fit the ring");
            store_tile_staged<FM, FN>(ep, m0 + wave_m * TM, n0 + wave_n * TN, acc, smem + wave * REG);
            return;
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                store_quad(ep, mb + fm * 16, nb + fn * 16, acc[fn][fm]);
        return;
    }
    constexpr uint32_t PART = BM * BN * 4;
    const auto rws = make_rsrc_u(g.ws + (size_t)t * g.split * (BM * BN), (uint32_t)(g.split * PART));
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            store16_coherent(rws, z * PART + (uint32_t)((((wave * FN + fn) * FM + fm) * 64 + lane) * 16),
                             acc[fn][fm]);
    if (!split_arrive_last(g.counters + t, g.split))
        return;
    // (as in mx_tile_kernel: a group's partials of a chunk requested
    // together, each element adding the chunks in z order)
    constexpr int FG = FM < 4 ? FM : 4;  // fragments per group
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int f0 = 0; f0 < FM; f0 += FG) {
            v4f sum[FG];
#pragma unroll
            for (int i = 0; i < FG; ++i)
                sum[i] = load16_coherent(rws, (uint32_t)((((wave * FN + fn) * FM + f0 + i) * 64 + lane) * 16));
            for (int zz = 1; zz < g.split; ++zz) {
                v4f part[FG];
#pragma unroll
                for (int i = 0; i < FG; ++i)
                    part[i] = load16_coherent(rws, zz * PART + (uint32_t)((((wave * FN + fn) * FM + f0 + i) * 64 + lane) * 16));
#pragma unroll
                for (int i = 0; i < FG; ++i)
                    sum[i] += part[i];
            }
#pragma unroll
            for (int i = 0; i < FG; ++i)
                store_quad(ep, mb + (f0 + i) * 16, nb + fn * 16, sum[i]);
        }
}

template <int BM, int BN, int WM, int WN, bool BPACK, bool SAPACK>
void launch_tile_deep(const GemmArgs &g, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((mx_tile_deep_kernel<BM, BN, WM, WN, BPACK, SAPACK>), dim3(grid), dim3(64 * WM * WN), 0, s, g);
}

#define MX_DEEP(BM, BN, WM, WN)                                                                   \
    template void launch_tile_deep<BM, BN, WM, WN, false, false>(const GemmArgs &, int, hipStream_t); \
    template void launch_tile_deep<BM, BN, WM, WN, true, false>(const GemmArgs &, int, hipStream_t);  \
    template void launch_tile_deep<BM, BN, WM, WN, true, true>(const GemmArgs &, int, hipStream_t);
MX_DEEP(256, 256, 2, 4)
MX_DEEP(256, 128, 2, 2)
MX_DEEP(128, 128, 2, 2)
MX_DEEP(64, 64, 2, 2)
#undef MX_DEEP

}  // namespace mx

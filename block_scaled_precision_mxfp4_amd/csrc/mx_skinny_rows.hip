// Skinny MXFP4 GEMM for 16 < M <= 64 on gfx950, waves splitting the rows of B.
//
// The single-wave-group skinny kernel (mx_skinny.hip) splits a workgroup's
// K chunk over its four waves, so every wave reads all M rows of A for its
// quarter of K, and A is read from L2 once per 16*NR rows of B.  At M = 64
// that A traffic equals the B stream itself.  Here the four waves of a
// workgroup share one K chunk and own different rows of B (16*NRW each):
// each batch's A rows are loaded once per workgroup into LDS with whole-line
// direct-to-LDS loads (2 or 4 rows x the batch's bytes per instruction,
// XOR-swizzled per 16-row group) and read by all four waves, while each wave
// streams its own B rows.  A workgroup covers 4x more rows of B for the same
// A bytes, and no cross-wave reduction is needed: each wave stores its own
// columns of D.
//
// Batches of U 128-K steps rotate through a ring of LDS slots; one barrier
// per batch hands a slot over.  A scales (row-major, 16-byte aligned rows)
// are staged the same way; other scale layouts are loaded by each wave.
// Row-major B goes through a wave-private part of the same slot: each load
// instruction covers whole 128-byte lines (4 rows x the batch's 256 bytes)
// instead of 64-byte halves of 16 rows, which the load path serves at a
// fraction of the whole-line rate; packed B (1 KiB contiguous per operand)
// is loaded straight into registers.
//
// A of a wider format (AFMT 1, 2: FP8 E4M3 / BF8 E5M2; 3, 4: FP6 E2M3 /
// E3M2; B stays FP4, "CDNA4 dense MFMA builtins", "Mixed-precision with
// scaling") is staged the same way, its rows of the batch being 8U or 6U
// 16-byte chunks (dense FP6: 24 bytes per K-block) in 32-slot LDS rows.  A
// lane's operand for K-block g of a step: FP8, the two 16-element runs K
// 16g.. and 64+16g.. of the step (two 16-byte reads); FP6, the block's 24
// bytes (three 8-byte reads).
#include "mx_args.hpp"
#include "mx_device.hpp"
#include "mx_pipe.hpp"

#include <type_traits>

namespace mx {

// SAM: 0 = row-major A scales staged in LDS (16-byte aligned rows, K-block
// count a multiple of 16); 1 = row-major A scales loaded per wave (any
// alignment); 2 = packed A scales loaded per wave (FP4 A only).
// U: 128-K steps per batch; NS: ring slots (NS - 1 batches in flight).
// AFMT: A's format (0 FP4, 1 FP8 E4M3, 2 BF8 E5M2, 3 FP6 E2M3, 4 FP6 E3M2);
// FP6 needs an even K-block count (chunks then never straddle the K end).
template <int MG, int NRW, int U, int NS, bool BPACK, bool SVEC, int SAM, int AFMT>
__global__ void __launch_bounds__(256) mx_rows_kernel(GemmArgs g)
{
    static_assert(U % 4 == 0 && NS >= 2, "whole 4-step scale groups per batch");
    static_assert(AFMT == 0 || SAM != 2, "wider A with row-major A scales");
    constexpr int G = U / 4;               // 4-step scale groups per batch
    constexpr int RW = 16 * NRW;           // B rows per wave
    constexpr int R = 4 * RW;              // B rows per workgroup
    constexpr int AR = MG * 16;            // A rows staged
    constexpr int AW = kFmtBits[AFMT];     // A element bits = dwords of a lane's operand
    constexpr int AKB = 4 * AW;            // bytes of one A K-block
    constexpr int ACU = U * AW;            // 16-byte chunks of an A row per batch
    constexpr int CPR = ACU <= 16 ? 16 : 32;  // LDS slots per A row (FP6: 24 of 32 used)
    static_assert(ACU <= CPR, "a batch's A row fits its LDS slots");
    constexpr int RPI = 64 / CPR;          // A rows per 1 KiB load instruction
    constexpr int A_BYTES = AR * CPR * 16;
    static_assert(A_BYTES % 4096 == 0, "the A stage splits evenly over the four waves");
    constexpr int A_DMA = A_BYTES / 4096;  // load instructions per wave per batch
    constexpr int SA_BYTES = AR * U * 4;   // row-major A scale bytes per batch
    constexpr int SA_ALLOC = SAM == 0 ? (SA_BYTES + 1023) / 1024 * 1024 : 16;
    constexpr int SA_PARTS = SAM == 0 ? SA_ALLOC / 1024 : 1;  // 1 KiB loads of the A scale stage
    static_assert(SA_ALLOC <= 4096, "one 16-byte lane per A scale chunk");
    constexpr bool BST = !BPACK;           // row-major B staged in LDS
    constexpr int CPB = U * 4;             // 16-byte chunks of a B row per batch
    constexpr int RPB = 64 / CPB;          // B rows per 1 KiB load instruction
    constexpr int B_WAVE = RW * CPB * 16;  // a wave's B bytes per batch
    constexpr int B_SLOT = BST ? 4 * B_WAVE : 0;
    __shared__ __attribute__((aligned(1024))) uint8_t s_a[NS * A_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t s_sa[NS * SA_ALLOC];
    __shared__ __attribute__((aligned(1024))) uint8_t s_b[BST ? NS * B_SLOT : 16];

    // memory instructions one batch issues per wave: a later batch's loads
    // may stay in flight while the wave waits for an earlier one
    constexpr int LN = A_DMA + U * NRW + (SAM == 0 ? 1 : SAM == 1 ? G * MG * 4 : (U / 2) * MG) +
                       (BPACK ? (U / 2) * NRW : G * NRW * (SVEC ? 1 : 4));
    constexpr int WN = (NS - 2) * LN < 63 ? (NS - 2) * LN : 63;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int z = blockIdx.x / g.tiles_n;
    const int t = blockIdx.x - z * g.tiles_n;
    const int n0 = t * R + wave * RW;  // this wave's first row of B (column of D)

    const int kb_begin = z * g.kb_per_split;
    const int kb_end = min(g.KB, kb_begin + g.kb_per_split);
    const int nb = (kb_end - kb_begin + 4 * U - 1) / (4 * U);  // batches (chunks are multiples of 16 blocks)

    const auto ra = make_rsrc_u(g.A, (uint32_t)(g.M * g.lda_b));
    const auto rsa = SAM == 2 ? make_rsrc_u(g.SA, (uint32_t)((g.M + 31) / 32 * g.sn8 * 256))
                              : make_rsrc_u(g.SA, (uint32_t)(g.M * g.ldsa));
    __amdgpu_buffer_rsrc_t rb, rsb;
    int half0 = 0;  // packed B scales: which 16-row half of its 32-row group row n0 is
    if constexpr (BPACK) {
        const int n16 = n0 / 16, g16 = max(0, min(NRW, (g.N + 15) / 16 - n16));
        rb = make_rsrc_u(g.B + (int64_t)n16 * g.ks_total * 1024, (uint32_t)(g16 * g.ks_total * 1024));
        const int n32 = n0 / 32;
        const int g32 = max(0, min((n0 + RW + 31) / 32 - n32, (g.N + 31) / 32 - n32));
        rsb = make_rsrc_u(g.SB + (int64_t)n32 * g.sn8 * 256, (uint32_t)(g32 * g.sn8 * 256));
        half0 = n16 & 1;
    } else {
        const int rows = max(0, min(RW, g.N - n0));
        rb = make_rsrc_u(g.B + (int64_t)n0 * g.ldb_b, (uint32_t)(rows * g.ldb_b));
        rsb = make_rsrc_u(g.SB + (int64_t)n0 * g.ldsb, (uint32_t)(rows * g.ldsb));
    }

    // one batch's per-wave loads
    struct Regs {
        v4i b[BST ? 1 : U][NRW];
        uint32_t sbp[BPACK ? U / 2 : 1][NRW];  // packed B scales: one word per step pair
        v4i sbr[BPACK ? 1 : G][NRW];           // row-major B scales: raw 4-step groups
        uint32_t sap[SAM == 2 ? U / 2 : 1][MG];
        v4i sar[SAM == 1 ? G : 1][MG];
    };

    auto issue = [&](int bi, auto slotc, Regs &r) __attribute__((always_inline)) {
        constexpr int SLOT = decltype(slotc)::value;
        const int kb0 = kb_begin + bi * 4 * U;  // first K-block of the batch (a multiple of 16)
        const int kbe = bi < nb ? kb_end : 0;   // batches past the chunk load nothing
        // A stage: whole 128-byte lines; slot s of row r holds chunk s ^ (r % 16)
        // of the row's batch (chunk c starts in K-block c * 16 / AKB; FP6
        // slots past the 6U chunks load nothing)
        uint8_t *da = s_a + SLOT * A_BYTES;
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            const int q = i * 4 + wave;  // 1 KiB instruction of the stage
            const int row = q * RPI + lane / CPR;
            const int c = (lane % CPR) ^ (row & 15);
            const bool ok = c < ACU && kb0 + c * 16 / AKB < kbe;
            load16_to_lds(ra, (lds_void *)(da + q * 1024),
                          ok ? (uint32_t)(row * g.lda_b + kb0 * AKB + c * 16) : kOOB);
        }
        if constexpr (SAM == 0) {
            // [AR][U*4] scale bytes, one 16-byte lane each (a lane past the
            // stage still writes zeros, inside the 1 KiB-rounded buffer).
            // Every wave loads one 1 KiB part, so that all waves issue the
            // same number of loads; waves that share a part write identical
            // bytes to the same place.
            uint8_t *ds = s_sa + SLOT * SA_ALLOC;
            const int part = wave % SA_PARTS;
            const int q = part * 64 + lane;
            const int row = q / (U / 4), kb = kb0 + (q % (U / 4)) * 16;
            load16_to_lds(rsa, (lds_void *)(ds + part * 1024),
                          row < AR && kb < kbe ? (uint32_t)(row * g.ldsa + kb) : kOOB);
        } else if constexpr (SAM == 1) {
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
#pragma unroll
                for (int mg = 0; mg < MG; ++mg)
                    r.sar[gi][mg] = load_scale_raw<false>(rsa, g.ldsa, mg * 16 + (lane & 15), kb0 + gi * 16, kbe, lane);
        } else {
#pragma unroll
            for (int p = 0; p < U / 2; ++p) {
                const int ks = kb0 / 4 + 2 * p;  // even: the word holds steps ks, ks+1 x both row halves
#pragma unroll
                for (int mg = 0; mg < MG; ++mg)
                    r.sap[p][mg] =
                        load4(rsa, ks * 4 < kbe ? (uint32_t)((((mg >> 1) * g.sn8 + (ks >> 1)) * 64 + lane) * 4) : kOOB);
            }
        }
        // this wave's rows of B and their scales
        if constexpr (BST) {
            // RPB rows x the batch's CPB chunks per instruction; slot s of
            // row r holds the row's chunk (K-block of the batch) s ^ (r % 16)
            uint8_t *db = s_b + SLOT * B_SLOT + wave * B_WAVE;
#pragma unroll
            for (int i = 0; i < RW / RPB; ++i) {
                const int row = i * RPB + lane / CPB;
                const int kb = kb0 + ((lane % CPB) ^ (row & 15));
                load16_to_lds_stream(rb, (lds_void *)(db + i * 1024),
                                     kb < kbe ? (uint32_t)(row * g.ldb_b + kb * 16) : kOOB);
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int ks = kb0 / 4 + u;
                const bool ok = ks * 4 + (lane >> 4) < kbe;
#pragma unroll
                for (int nr = 0; nr < NRW; ++nr)
                    r.b[u][nr] = load16_stream(rb, ok ? (uint32_t)(((nr * g.ks_total + ks) * 64 + lane) * 16) : kOOB);
            }
        }
        if constexpr (BPACK) {
#pragma unroll
            for (int p = 0; p < U / 2; ++p) {
                const int ks = kb0 / 4 + 2 * p;
#pragma unroll
                for (int nr = 0; nr < NRW; ++nr) {
                    const int grp = (half0 + nr) >> 1;
                    r.sbp[p][nr] =
                        load4(rsb, ks * 4 < kbe ? (uint32_t)(((grp * g.sn8 + (ks >> 1)) * 64 + lane) * 4) : kOOB);
                }
            }
        } else {
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
#pragma unroll
                for (int nr = 0; nr < NRW; ++nr)
                    r.sbr[gi][nr] = load_scale_raw<SVEC>(rsb, g.ldsb, nr * 16 + (lane & 15), kb0 + gi * 16, kbe, lane);
        }
    };

    v4f acc[NRW][MG];
#pragma unroll
    for (int nr = 0; nr < NRW; ++nr)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
            acc[nr][mg] = v4f{0.f, 0.f, 0.f, 0.f};

    // LDS reads go through asm with explicit waits: the compiler would make
    // every read wait for all direct-to-LDS loads in flight, other slots'
    // included, and drain the ring
    const uint32_t a_base = lds_addr(s_a) + (uint32_t)((lane & 15) * CPR * 16);
    const uint32_t sa_base = lds_addr(s_sa) + (uint32_t)((lane & 15) * U * 4);
    const uint32_t b_base = lds_addr(s_b) + (uint32_t)(wave * B_WAVE + (lane & 15) * CPB * 16);
    auto compute = [&](auto slotc, const Regs &r) __attribute__((always_inline)) {
        constexpr int SLOT = decltype(slotc)::value;
        uint32_t saw[G][MG];
        if constexpr (SAM == 0) {
            v4i sv[G][MG];
            static_for<G>([&](auto gc) {
                static_for<MG>([&](auto mc) {
                    constexpr int OFF = SLOT * SA_ALLOC + decltype(mc)::value * 16 * U * 4 + decltype(gc)::value * 16;
                    sv[gc.value][mc.value] = lds_read16<OFF>(sa_base);
                });
            });
            lds_wait_n<0>(sv);
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
#pragma unroll
                for (int mg = 0; mg < MG; ++mg)
                    saw[gi][mg] = scale_group_word<true>(sv[gi][mg], lane);
        } else if constexpr (SAM == 1) {
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
#pragma unroll
                for (int mg = 0; mg < MG; ++mg)
                    saw[gi][mg] = scale_group_word<false>(r.sar[gi][mg], lane);
        }
        // staged B: this wave's fragments of the whole batch, read first
        // (row nr*16 + lane%16, chunk 4u + lane/16 at slot chunk ^ (row % 16))
        v4i bst[BST ? U : 1][NRW];
        if constexpr (BST) {
            const uint32_t bslot = b_base + (uint32_t)(SLOT * B_SLOT);
            static_for<U>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                const uint32_t a = bslot + (uint32_t)((((u * 4) + (lane >> 4)) ^ (lane & 15)) * 16);
                static_for<NRW>([&](auto nc) {
                    constexpr int nr = decltype(nc)::value;
                    bst[u][nr] = lds_read16<nr * 16 * CPB * 16>(a);
                });
            });
        }
        // A fragments of step u, row mg*16 + lane%16, K-block g = lane/16 of
        // the step, each 16-byte chunk c at slot c ^ (row % 16): FP4 chunk
        // 4u + g; FP8 chunks 8u + g and 8u + g + 4; FP6 the 8-byte pieces at
        // bytes 96u + 24g + 8j, j = 0..2.  One step is read ahead of the
        // multiplies.
        const uint32_t slot_base = a_base + SLOT * A_BYTES;
        constexpr int NA = AW == 4 ? 1 : AW == 8 ? 2 : 3;  // reads per fragment
        struct AStep {
            v4i x[AW == 6 ? 1 : NA][MG];
            v2u y[AW == 6 ? NA : 1][MG];
        };
        AStep af[2];
        auto read_step = [&](auto uc, AStep &dst) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value;
            const int gq = lane >> 4, row = lane & 15;
            if constexpr (AW == 6) {
                static_for<NA>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    const int byte = 24 * gq + 8 * j;  // within the step's 96 bytes
                    const uint32_t a =
                        slot_base + (uint32_t)((((u * 6) + (byte >> 4)) ^ row) * 16 + (byte & 8));
                    static_for<MG>([&](auto mc) {
                        dst.y[j][mc.value] = lds_read8<decltype(mc)::value * 16 * CPR * 16>(a);
                    });
                });
            } else {
                static_for<NA>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    const uint32_t a = slot_base + (uint32_t)((((u * 4 * NA) + gq + 4 * j) ^ row) * 16);
                    static_for<MG>([&](auto mc) {
                        dst.x[j][mc.value] = lds_read16<decltype(mc)::value * 16 * CPR * 16>(a);
                    });
                });
            }
        };
        auto wait_step = [&](auto nc, AStep &st) __attribute__((always_inline)) {
            if constexpr (AW == 6)
                lds_wait_n<decltype(nc)::value>(st.y);
            else
                lds_wait_n<decltype(nc)::value>(st.x);
        };
        read_step(std::integral_constant<int, 0>{}, af[0]);
        static_for<U>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            if constexpr (u == 0 && BST)
                lds_wait_n<NA * MG>(bst);  // the B reads went out before step 0's
            if constexpr (u + 1 < U) {
                read_step(std::integral_constant<int, u + 1>{}, af[(u + 1) & 1]);
                wait_step(std::integral_constant<int, NA * MG>{}, af[u & 1]);
            } else {
                wait_step(std::integral_constant<int, 0>{}, af[u & 1]);
            }
            const AStep &cur = af[u & 1];
#pragma unroll
            for (int nr = 0; nr < NRW; ++nr)
#pragma unroll
                for (int mg = 0; mg < MG; ++mg) {
                    // packed words: this row half's bytes shifted to 0 and 2
                    const int ob = BPACK ? (u & 1) * 2 : (u & 3);
                    const uint32_t sbr = BPACK ? r.sbp[u / 2][nr] >> (8 * ((half0 + nr) & 1))
                                               : scale_group_word<SVEC>(r.sbr[u / 4][nr], lane);
                    const int oa = SAM == 2 ? (u & 1) * 2 : (u & 3);
                    const uint32_t sar = SAM == 2 ? r.sap[u / 2][mg] >> (8 * (mg & 1)) : saw[u / 4][mg];
                    const v4i bf = BST ? bst[BST ? u : 0][nr] : r.b[BST ? 0 : u][nr];
                    if constexpr (AW == 4) {
                        acc[nr][mg] = mma_sel(ob, oa, bf, cur.x[0][mg], acc[nr][mg], (int)sbr, (int)sar);
                    } else {
                        v8i a;
                        if constexpr (AW == 8) {
                            const v4i lo = cur.x[0][mg], hi = cur.x[1][mg];
                            a = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        } else {
                            const v2u p0 = cur.y[0][mg], p1 = cur.y[1][mg], p2 = cur.y[2][mg];
                            a = v8i{(int)p0[0], (int)p0[1], (int)p1[0], (int)p1[1], (int)p2[0], (int)p2[1], 0, 0};
                        }
                        acc[nr][mg] = mma_sel_wide<kFmtHw[AFMT]>(ob, oa, bf, a, acc[nr][mg], (int)sbr, (int)sar);
                    }
                }
        });
    };

    // batch b's loads have landed in every wave (at most NS - 2 later
    // batches still in flight) and every wave is done with the slot the next
    // issue overwrites
    auto hand_over = [&]() __attribute__((always_inline)) {
        wait_vmcnt<WN>();  // a real wait instruction: the compiler counts it
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // ring of NS slots: batch b lives in slot b % NS; the loop is unrolled
    // NS times so that every slot and register set is a compile-time choice
    Regs r[NS];
    static_for<NS - 1>([&](auto jc) { issue(jc.value, jc, r[jc.value]); });
    hand_over();
    // The issue of every step is unconditional (past the chunk it loads
    // nothing and writes zeros into a slot no wave reads again): a register
    // set assigned on only one path would become a merge point that the
    // compiler resolves with a copy, and a copy waits for its load.  The
    // slot an issue overwrites was last read by the step before it, which
    // ended with a barrier if it ran at all.
    for (int bi = 0; bi < nb; bi += NS) {
        static_for<NS>([&](auto jc) {
            constexpr int J = decltype(jc)::value;
            constexpr int NXT = (J + NS - 1) % NS;
            issue(bi + J + NS - 1, std::integral_constant<int, NXT>{}, r[NXT]);
            if (bi + J < nb) {
                compute(jc, r[J]);
                hand_over();
            }
        });
    }
    wait_vmcnt<0>();  // loads issued past the chunk (they write zeros into free slots)

    // ---- epilogue: each wave owns its columns
    Epilogue ep{g.D, g.C, g.alpha, g.beta, g.M, g.N, g.ldd, g.ldc, g.d_vec, g.c_vec, g.c_f32};
    const int mb = lane & 15, nb4 = n0 + 4 * (lane >> 4);
    if (g.split == 1) {
#pragma unroll
        for (int nr = 0; nr < NRW; ++nr)
#pragma unroll
            for (int mg = 0; mg < MG; ++mg)
                store_quad(ep, mb + mg * 16, nb4 + nr * 16, acc[nr][mg]);
        return;
    }
    // fp32 partials of this chunk: [tile][z][wave][nr][mg][lane] float4s
    constexpr uint32_t PART = 4 * NRW * MG * 64 * 16;  // bytes per workgroup partial
    const auto rws = make_rsrc_u(g.ws + (size_t)t * g.split * (PART / 4), (uint32_t)(g.split * PART));
#pragma unroll
    for (int nr = 0; nr < NRW; ++nr)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
            store16_coherent(rws, z * PART + (uint32_t)((((wave * NRW + nr) * MG + mg) * 64 + lane) * 16), acc[nr][mg]);
    if (!split_arrive_last(g.counters + t, g.split))
        return;
    // every fragment's partial of a chunk is requested before any is added,
    // so that one memory latency per chunk is paid, not one per fragment;
    // each element still adds the chunks in z order
    v4f sum[NRW][MG];
#pragma unroll
    for (int nr = 0; nr < NRW; ++nr)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
            sum[nr][mg] = load16_coherent(rws, (uint32_t)((((wave * NRW + nr) * MG + mg) * 64 + lane) * 16));
    for (int zz = 1; zz < g.split; ++zz) {
        v4f part[NRW][MG];
#pragma unroll
        for (int nr = 0; nr < NRW; ++nr)
#pragma unroll
            for (int mg = 0; mg < MG; ++mg)
                part[nr][mg] = load16_coherent(rws, zz * PART + (uint32_t)((((wave * NRW + nr) * MG + mg) * 64 + lane) * 16));
#pragma unroll
        for (int nr = 0; nr < NRW; ++nr)
#pragma unroll
            for (int mg = 0; mg < MG; ++mg)
                sum[nr][mg] += part[nr][mg];
    }
#pragma unroll
    for (int nr = 0; nr < NRW; ++nr)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
            store_quad(ep, mb + mg * 16, nb4 + nr * 16, sum[nr][mg]);
}

template <int MG, int NRW, int U, int NS, bool BPACK, int AFMT>
static void launch_rows(const GemmArgs &g, int grid, hipStream_t s)
{
    // A-scale source: packed words (FP4 A), 16-byte aligned row groups
    // staged in LDS, or per-wave byte loads; B scales: 16-byte groups when
    // aligned
    if constexpr (BPACK) {
        if constexpr (AFMT == 0) {
            if (g.sa_packed) {
                hipLaunchKernelGGL((mx_rows_kernel<MG, NRW, U, NS, true, true, 2, 0>), dim3(grid), dim3(256), 0, s, g);
                return;
            }
        }
        if (g.sa16)
            hipLaunchKernelGGL((mx_rows_kernel<MG, NRW, U, NS, true, true, 0, AFMT>), dim3(grid), dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((mx_rows_kernel<MG, NRW, U, NS, true, true, 1, AFMT>), dim3(grid), dim3(256), 0, s, g);
    } else {
        if (g.sa16) {
            if (g.sb16)
                hipLaunchKernelGGL((mx_rows_kernel<MG, NRW, U, NS, false, true, 0, AFMT>), dim3(grid), dim3(256), 0, s, g);
            else
                hipLaunchKernelGGL((mx_rows_kernel<MG, NRW, U, NS, false, false, 0, AFMT>), dim3(grid), dim3(256), 0, s,
                                   g);
        } else {
            if (g.sb16)
                hipLaunchKernelGGL((mx_rows_kernel<MG, NRW, U, NS, false, true, 1, AFMT>), dim3(grid), dim3(256), 0, s, g);
            else
                hipLaunchKernelGGL((mx_rows_kernel<MG, NRW, U, NS, false, false, 1, AFMT>), dim3(grid), dim3(256), 0, s,
                                   g);
        }
    }
}

// Batch and ring shape per A format: FP4 A takes U4 steps per batch in NS4
// slots; a wider A four steps per batch in NSW slots (A's 32-slot rows, B
// and the A scales then fill 123-147 KiB of LDS).  The lean entry (FP4 A,
// row-major B, two slots: 66 KiB at four steps) lets two workgroups share a
// CU when the grid has more workgroups than CUs.
#define MX_ROWS(MG, NRW, U4, NS4, NSW)                                                                            \
    {MG, NRW,                                                                                                  \
     {launch_rows<MG, NRW, U4, NS4, false, 0>, launch_rows<MG, NRW, 4, NSW, false, 1>,                         \
      launch_rows<MG, NRW, 4, NSW, false, 2>, launch_rows<MG, NRW, 4, NSW, false, 3>,                          \
      launch_rows<MG, NRW, 4, NSW, false, 4>},                                                                 \
     {launch_rows<MG, NRW, U4, NS4, true, 0>, launch_rows<MG, NRW, 4, NSW, true, 1>,                           \
      launch_rows<MG, NRW, 4, NSW, true, 2>, launch_rows<MG, NRW, 4, NSW, true, 3>,                            \
      launch_rows<MG, NRW, 4, NSW, true, 4>},                                                                  \
     {"rows_m" #MG "x16_n4x" #NRW "x16_u" #U4 "_r" #NS4, "rows_fp8_m" #MG "x16_n4x" #NRW "x16_u4_r" #NSW,      \
      "rows_bf8_m" #MG "x16_n4x" #NRW "x16_u4_r" #NSW, "rows_fp6_m" #MG "x16_n4x" #NRW "x16_u4_r" #NSW,       \
      "rows_fp6_m" #MG "x16_n4x" #NRW "x16_u4_r" #NSW},                                                   \
     launch_rows<MG, NRW, U4, 2, false, 0>, "rows_m" #MG "x16_n4x" #NRW "x16_u" #U4 "_r2"}
const RowsKernel *rows_kernels(int *count)
{
    static const RowsKernel table[] = {
        MX_ROWS(2, 1, 4, 4, 4), MX_ROWS(3, 1, 4, 4, 3), MX_ROWS(4, 1, 4, 4, 3),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}
#undef MX_ROWS

}  // namespace mx

// Skinny MXFP4 GEMM for M <= 16 (decode / GEMV shapes) on gfx950.
//
// Here the whole cost is reading B once from HBM, so the kernel streams B
// straight from memory into registers (16 bytes per lane, one instruction
// operand per 16 rows x 128 K) with several loads in flight per lane, and
// keeps the tiny A in the L2.  A workgroup owns 16*NR rows of B (= columns
// of D) and one K chunk; its four waves take consecutive quarters of that
// chunk and add their accumulators through LDS in a fixed order.  The
// accumulators of a wave cover all M <= 16*MG rows of D (the table holds
// MG = 1: for 16 < M <= 64 every wave would re-read all of A for its
// quarter of K, and the rows kernel, which shares A through LDS, is
// faster).  The scaled FP4
// instruction does the arithmetic: rows of A past M are zero lanes
// (out-of-range loads return zero without memory traffic), which costs
// nothing here because the matrix unit is far from busy at HBM speed.
//
// Split K across workgroups (more workgroups than row blocks, to keep
// enough bytes in flight) combines fp32 partials in a fixed order in the
// last workgroup to arrive, in the same launch.
#include "mx_args.hpp"
#include "mx_device.hpp"
#include "mx_quantize.hpp"
#include "mx_pipe.hpp"

#include <type_traits>

namespace mx {

// A1: A is a single row (M == 1, row-major scales).  Each wave then loads
// the row's K-blocks of a whole batch with one instruction (lane l: K-block
// l of the batch, with its scale byte) instead of one mostly-empty fragment
// load per step, and forms each step's operand with cross-lane permutes:
// operand lane l takes K-block 4u + l/16 of step u.  Operand lanes of rows
// 1..15 then carry row 0's values too; their result rows are never stored.
// AFMT: A's format (0 FP4; 1 FP8 E4M3, 2 BF8 E5M2, 3 FP6 E2M3, 4 FP6 E3M2;
// B is FP4).  A lane's operand is 32 elements of its row, 16, 32 or 24
// bytes held as 4, 8 or 6 dwords.  For the 4- and 6-bit formats they are
// K-block g = lane/16 of the 128-K step.  For the 8-bit formats the
// instruction reads the 32 bytes as two runs of 16 elements, K 16g..16g+15
// and 64+16g..64+16g+15 of the step (found with an identity-B probe on
// MI355X; the scales still go by 32-element block, lane g holding block
// g's), so the lane loads those two 16-byte pieces.
// AFMT kBf16A: A is a single bf16 row (g.A, g.lda_b bytes per row), quantized
// to MXFP4 on load with the activation quantizer's rule; g.SA is not read.
constexpr int kBf16A = 5;

template <int MG, int NR, bool BPACK, bool SVEC, bool APACK, bool A1, int AFMT = 0>
__global__ void __launch_bounds__(256) mx_skinny_kernel(GemmArgs g)
{
    static_assert(!A1 || (MG == 1 && !APACK), "single-row A: one row group, row-major scales");
    constexpr bool XQ = AFMT == kBf16A;  // bf16 A, quantized on load
    static_assert(!XQ || A1, "quantize-on-load needs the single-row path");
    constexpr int AF = XQ ? 0 : AFMT;   // the operand format the instruction sees
    constexpr int AW = kFmtBits[AF];    // dwords of a lane's A operand (= element bits)
    constexpr int AKB = 4 * AW;         // bytes of one A K-block
    constexpr bool A8 = AW == 8;        // 8-bit A: two 16-element runs per lane
    using a_t = typename std::conditional<AF == 0, v4i, v8i>::type;
    // A1 with 8-bit A holds one 16-byte chunk per lane, else one K-block
    using aw_t = typename std::conditional<A8, v4i, a_t>::type;
    static_assert(!(A1 && A8) || (NR + MG) <= 3, "single-row 8-bit A: 8 steps per batch, one chunk per lane");
    // one lane's K-block of A at byte offset off (out-of-range offsets read zeros)
    auto load_a = [](__amdgpu_buffer_rsrc_t r, uint32_t off) __attribute__((always_inline)) {
        if constexpr (AF == 0) {
            return load16(r, off);
        } else {
            const v4i lo = load16(r, off);
            v8i a = {lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
            if constexpr (AW == 8) {
                const v4i hi = load16(r, off == kOOB ? kOOB : off + 16);
                a[4] = hi[0], a[5] = hi[1], a[6] = hi[2], a[7] = hi[3];
            } else {
                const v2u hi = load8(r, off == kOOB ? kOOB : off + 16);
                a[4] = (int)hi[0], a[5] = (int)hi[1];
            }
            return a;
        }
    };
    constexpr int R = 16 * NR;                      // B rows per workgroup
    constexpr int NF = NR * MG;                     // 16x16 result blocks per workgroup
    // 128-K steps per batch (two batches in flight): four, except the
    // single-row 8-bit A, whose batch is one 16-byte chunk per lane (eight
    // steps).  Four-step batches start the multiplies earlier and measured
    // faster than eight-step ones on MI355X (16x4096x4096: 6.0 -> 5.4 us,
    // 1x28672x8192: 22.8 -> 21.5 us; 1x8192x8192 unchanged).
    constexpr int U = A1 && A8 ? 8 : 4;
    constexpr int G = U / 4;                        // scale groups (4 steps) per batch
    __shared__ v4f s_red[4][NF][64];
    // Row-major B with a single-row A: B goes through a wave-private LDS
    // buffer per batch so that every load instruction covers whole 128-byte
    // lines (a row's U*64 bytes of the batch, RPI rows per instruction) instead of
    // 64-byte halves of 16 rows; 16-byte chunk c of row r sits at slot
    // c ^ (r % 16), so a fragment's 16 rows hit 16 different bank groups.
    constexpr bool BST = A1 && !BPACK;
    constexpr int CPR = U * 4;  // 16-byte chunks per row per batch
    constexpr int BST_BYTES = BST ? NR * 16 * CPR * 16 : 16;
    __shared__ __attribute__((aligned(1024))) uint8_t s_bst0[4][BST_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t s_bst1[4][BST_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // no XCD regrouping here: workgroups share no B, and spreading each XCD's
    // streams over the whole matrix (consecutive workgroups on different
    // XCDs) measured faster than giving each XCD one contiguous part
    const int lg = blockIdx.x;
    const int z = lg / g.tiles_n;
    const int t = lg - z * g.tiles_n;
    const int n0 = t * R;  // first row of B (column of D) of this workgroup

    // K range: chunks are multiples of 16 K-blocks, wave ranges multiples of 4 steps
    const int kb_begin = z * g.kb_per_split;
    const int kb_end = min(g.KB, kb_begin + g.kb_per_split);
    const int ks_begin = kb_begin >> 2, ks_end = (kb_end + 3) >> 2;
    const int q = (((ks_end - ks_begin + 3) >> 2) + 3) & ~3;  // steps per wave
    const int w_begin = ks_begin + wave * q;
    const int w_end = min(ks_end, w_begin + q);
    const int kb_wend = min(kb_end, w_end * 4);  // K-blocks this wave may touch

    const auto ra = make_rsrc_u(g.A, (uint32_t)(g.M * g.lda_b));
    const auto rsa = APACK ? make_rsrc_u(g.SA, (uint32_t)((g.M + 31) / 32 * g.sn8 * 256))
                           : make_rsrc_u(g.SA, (uint32_t)(g.M * g.ldsa));
    __amdgpu_buffer_rsrc_t rb, rsb;
    int half0 = 0;  // packed scales: which 16-row half of its 32-row group row n0 is
    if constexpr (BPACK) {
        const int n16 = n0 / 16, g16 = max(0, min(NR, (g.N + 15) / 16 - n16));
        rb = make_rsrc_u(g.B + (int64_t)n16 * g.ks_total * 1024, (uint32_t)(g16 * g.ks_total * 1024));
        const int n32 = n0 / 32;
        const int g32 = max(0, min((n0 + R + 31) / 32 - n32, (g.N + 31) / 32 - n32));
        rsb = make_rsrc_u(g.SB + (int64_t)n32 * g.sn8 * 256, (uint32_t)(g32 * g.sn8 * 256));
        half0 = n16 & 1;
    } else {
        const int rows = max(0, min(R, g.N - n0));
        rb = make_rsrc_u(g.B + (int64_t)n0 * g.ldb_b, (uint32_t)(rows * g.ldb_b));
        rsb = make_rsrc_u(g.SB + (int64_t)n0 * g.ldsb, (uint32_t)(rows * g.ldsb));
    }

    struct Batch {
        v4i b[U][NR];
        a_t a[A1 ? 1 : U][MG];
        // scales as loaded: packed, one word per step pair (both row halves);
        // row-major, one raw 16-byte group per 4 steps
        uint32_t sbp[BPACK ? U / 2 : 1][NR];
        v4i sbr[BPACK ? 1 : G][NR];
        uint32_t sap[APACK ? U / 2 : 1][MG];
        v4i sar[APACK || A1 ? 1 : G][MG];
        aw_t aw;       // A1: K-block kb0 + lane (8-bit A: 16-byte chunk lane) of row 0
        uint32_t saw;  // A1: its scale byte
        // XQ: bf16 quarter-blocks of the batch, U/4 loads of 64 lanes: in load
        // h, lane l holds elements 8(l%4) .. 8(l%4)+7 of K-block 16h + l/4
        v4i xq[XQ ? U / 4 : 1];
    };

    auto load_batch = [&](int ks0, Batch &bt, auto bufc) __attribute__((always_inline)) {
        if constexpr (BST) {
            uint8_t *dst = decltype(bufc)::value ? s_bst1[wave] : s_bst0[wave];
            constexpr int RPI = 64 / CPR;  // rows per 1 KiB instruction
            const int rl = lane / CPR, sl = lane % CPR;
#pragma unroll
            for (int i = 0; i < NR * 16 / RPI; ++i) {
                const int row = i * RPI + rl;
                const int kbc = ks0 * 4 + (sl ^ (row & 15));  // the chunk this slot holds
                load16_to_lds_stream(rb, (lds_void *)(dst + i * 1024),
                              kbc < kb_wend ? (uint32_t)(row * g.ldb_b + kbc * 16) : kOOB);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ks = ks0 + u;
            const int kb = ks * 4 + (lane >> 4);
            const bool ok = kb < kb_wend;
#pragma unroll
            for (int nr = 0; nr < NR; ++nr) {
                if constexpr (BST)
                    ;  // staged above
                else if constexpr (BPACK)
                    bt.b[u][nr] = load16_stream(rb, ok ? (uint32_t)(((nr * g.ks_total + ks) * 64 + lane) * 16) : kOOB);
                else
                    bt.b[u][nr] = load16_stream(rb, ok ? (uint32_t)((nr * 16 + (lane & 15)) * g.ldb_b + kb * 16) : kOOB);
            }
            if constexpr (!A1 && A8) {
                // bytes 16g..16g+15 (K-block 2*ks0.. first pair) and 64+16g.. of the step
                const int gq = lane >> 4;
                const bool ok_lo = ks * 4 + (gq >> 1) < kb_wend, ok_hi = ks * 4 + 2 + (gq >> 1) < kb_wend;
#pragma unroll
                for (int mg = 0; mg < MG; ++mg) {
                    const uint32_t base = (uint32_t)((mg * 16 + (lane & 15)) * g.lda_b + ks * 128 + gq * 16);
                    const v4i lo = load16(ra, ok_lo ? base : kOOB), hi = load16(ra, ok_hi ? base + 64 : kOOB);
                    bt.a[u][mg] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
            } else if constexpr (!A1) {
#pragma unroll
                for (int mg = 0; mg < MG; ++mg)
                    bt.a[u][mg] = load_a(ra, ok ? (uint32_t)((mg * 16 + (lane & 15)) * g.lda_b + kb * AKB) : kOOB);
            }
        }
        if constexpr (XQ) {
#pragma unroll
            for (int h = 0; h < U / 4; ++h) {
                const int kbx = ks0 * 4 + 16 * h + (lane >> 2);
                bt.xq[h] = load16(ra, kbx < kb_wend ? (uint32_t)(kbx * 64 + (lane & 3) * 16) : kOOB);
            }
        } else if constexpr (A1) {
            const int kbl = ks0 * 4 + lane;
            const bool okl = lane < 4 * U && kbl < kb_wend;
            if constexpr (A8) {
                // 16-byte chunk `lane` of the batch (K-block kb0 + lane/2)
                const bool okc = ks0 * 4 + (lane >> 1) < kb_wend;
                bt.aw = load16(ra, okc ? (uint32_t)(ks0 * 128 + lane * 16) : kOOB);
            } else {
                bt.aw = load_a(ra, okl ? (uint32_t)(kbl * AKB) : kOOB);
            }
            bt.saw = load1(rsa, okl ? (uint32_t)kbl : kOOB);
        }
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            const int kb0 = (ks0 + 4 * gi) * 4;  // first K-block of the group
            if constexpr (!APACK && !A1) {
#pragma unroll
                for (int mg = 0; mg < MG; ++mg)
                    bt.sar[gi][mg] = load_scale_raw<SVEC>(rsa, g.ldsa, mg * 16 + (lane & 15), kb0, kb_wend, lane);
            }
            if constexpr (!BPACK) {
#pragma unroll
                for (int nr = 0; nr < NR; ++nr)
                    bt.sbr[gi][nr] = load_scale_raw<SVEC>(rsb, g.ldsb, nr * 16 + (lane & 15), kb0, kb_wend, lane);
            }
        }
        if constexpr (APACK) {
#pragma unroll
            for (int p = 0; p < U / 2; ++p) {
                const int ks = ks0 + 2 * p;  // even: the word holds steps ks, ks+1 x both row halves
#pragma unroll
                for (int mg = 0; mg < MG; ++mg) {
                    const uint32_t w =
                        load4(rsa, ks * 4 < kb_wend ? (uint32_t)((((mg >> 1) * g.sn8 + (ks >> 1)) * 64 + lane) * 4) : kOOB);
                    bt.sap[p][mg] = w;
                }
            }
        }
        if constexpr (BPACK) {
#pragma unroll
            for (int p = 0; p < U / 2; ++p) {
                const int ks = ks0 + 2 * p;  // even: the word holds steps ks, ks+1 x both row halves
#pragma unroll
                for (int nr = 0; nr < NR; ++nr) {
                    const int grp = (half0 + nr) >> 1;
                    const uint32_t w =
                        load4(rsb, ks * 4 < kb_wend ? (uint32_t)(((grp * g.sn8 + (ks >> 1)) * 64 + lane) * 4) : kOOB);
                    bt.sbp[p][nr] = w;
                }
            }
        }
    };

    v4f acc[NR][MG];
#pragma unroll
    for (int nr = 0; nr < NR; ++nr)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
            acc[nr][mg] = v4f{0.f, 0.f, 0.f, 0.f};

    // vector-memory instructions of one load_batch (all lanes issue all of
    // them): staged B, the single A row and its scales, row-major B scales
    constexpr int LN = NR * U + (XQ ? U / 4 : AW == 6 ? 3 : 2) + G * NR * (SVEC ? 1 : 4);
    static_assert(!BST || LN < 64, "vmcnt range");
    auto compute = [&](const Batch &bt, auto bufc, auto lastc) __attribute__((always_inline)) {
        v4i bst[BST ? U : 1][NR];
        if constexpr (BST) {
            // this batch's staging loads have landed (the next batch's LN
            // loads may still be in flight, unless this is the last batch);
            // then all fragment reads at once
            if constexpr (decltype(lastc)::value)
                wait_vmcnt<0>();
            else
                wait_vmcnt<LN>();
            const uint32_t base = lds_addr(decltype(bufc)::value ? s_bst1[wave] : s_bst0[wave]) +
                                  (uint32_t)((lane & 15) * CPR * 16);
            static_for<U>([&](auto ui) {
                constexpr int u = decltype(ui)::value;
                const uint32_t a = base + (uint32_t)((((u * 4) + (lane >> 4)) ^ (lane & 15)) * 16);
                static_for<NR>([&](auto ni) {
                    constexpr int nr = decltype(ni)::value;
                    bst[u][nr] = lds_read16<nr * 16 * CPR * 16>(a);
                });
            });
            lds_wait_n<0>(bst);
        }
        // the single A row's K-blocks of the batch: lane b < 4U holds block
        // ks0*4 + b (16 bytes) and its scale byte
        aw_t aw_use = {};
        uint32_t saw_use = 0;
        if constexpr (XQ) {
            // quantize the quarter-blocks (four lanes per block), then gather
            // block b's four words and its scale from lanes 4(b%16) .. +3 of
            // load b/16
            const int src = (lane & 15) * 16;  // byte address of lane 4(b%16)
#pragma unroll
            for (int h = 0; h < U / 4; ++h) {
                uint32_t word;
                uint8_t sc;
                quantize_quarter(bt.xq[h], word, sc);
                const bool mine = (lane >> 4) == h;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int v = __builtin_amdgcn_ds_bpermute(src + 4 * i, (int)word);
                    aw_use[i] = mine ? v : aw_use[i];
                }
                const int sv = __builtin_amdgcn_ds_bpermute(src, (int)sc);
                saw_use = mine ? (uint32_t)sv : saw_use;
            }
        } else if constexpr (A1) {
            aw_use = bt.aw;
            saw_use = bt.saw;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            a_t a1 = {};
            uint32_t sa1 = 0;
            if constexpr (A1 && A8) {
                // chunks 8u + g and 8u + 4 + g of the batch
                const int lo = (8 * u + (lane >> 4)) * 4, hi = lo + 16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a1[i] = __builtin_amdgcn_ds_bpermute(lo, aw_use[i]);
                    a1[4 + i] = __builtin_amdgcn_ds_bpermute(hi, aw_use[i]);
                }
            }
            if constexpr (A1) {
                const int src = (4 * u + (lane >> 4)) * 4;  // byte address of the source lane
                if constexpr (!A8) {
#pragma unroll
                    for (int i = 0; i < AW; ++i)
                        a1[i] = __builtin_amdgcn_ds_bpermute(src, aw_use[i]);
                }
                sa1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)saw_use) & 0xFFu;
            }
#pragma unroll
            for (int nr = 0; nr < NR; ++nr)
#pragma unroll
                for (int mg = 0; mg < MG; ++mg) {
                    // packed words: this row half's bytes shifted to 0 and 2
                    const int ob = BPACK ? (u & 1) * 2 : (u & 3);
                    const uint32_t sbr = BPACK ? bt.sbp[u / 2][nr] >> (8 * ((half0 + nr) & 1))
                                               : scale_group_word<SVEC>(bt.sbr[u / 4][nr], lane);
                    const int oa = A1 ? 0 : APACK ? (u & 1) * 2 : (u & 3);
                    const uint32_t sar = A1      ? sa1
                                         : APACK ? bt.sap[u / 2][mg] >> (8 * (mg & 1))
                                                 : scale_group_word<SVEC>(bt.sar[u / 4][mg], lane);
                    const v4i bf = BST ? bst[BST ? u : 0][nr] : bt.b[u][nr];
                    if constexpr (AF == 0)
                        acc[nr][mg] = mma_sel(ob, oa, bf, A1 ? a1 : bt.a[u][mg], acc[nr][mg], (int)sbr, (int)sar);
                    else
                        acc[nr][mg] = mma_sel_wide<kFmtHw[AF]>(ob, oa, bf, A1 ? a1 : bt.a[u][mg], acc[nr][mg],
                                                                 (int)sbr, (int)sar);
                }
        }
    };

    // two batches in flight: issue the next before multiplying the current
    // (scheduling barriers keep each batch's loads ahead of the multiplies
    // of the previous one; left alone the scheduler sinks them below).  The
    // last pair of batches is peeled so that no batch past the wave's range
    // is issued: such a batch loads nothing, but its instructions still
    // queue on the load path ahead of the last multiplies (at M = 1 the
    // peel took the 1 x 8192 x 8192 GEMV from 9.5 to 8.9 us).  A wave with
    // an empty range multiplies two batches of zeros, which adds +0.
    using Buf0 = std::integral_constant<int, 0>;
    using Buf1 = std::integral_constant<int, 1>;
    using More = std::false_type;
    using Last = std::true_type;
    Batch cur, nxt;
    load_batch(w_begin, cur, Buf0{});
    int ks0 = w_begin;
    for (; ks0 + 2 * U < w_end; ks0 += 2 * U) {
        load_batch(ks0 + U, nxt, Buf1{});
        __builtin_amdgcn_sched_barrier(0);
        compute(cur, Buf0{}, More{});
        __builtin_amdgcn_sched_barrier(0);
        load_batch(ks0 + 2 * U, cur, Buf0{});
        __builtin_amdgcn_sched_barrier(0);
        compute(nxt, Buf1{}, More{});
        __builtin_amdgcn_sched_barrier(0);
    }
    load_batch(ks0 + U, nxt, Buf1{});
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, Buf0{}, More{});
    __builtin_amdgcn_sched_barrier(0);
    compute(nxt, Buf1{}, Last{});

    // ---- the four waves' sums, added in wave order; wave w then owns blocks f = w, w+4, ...
#pragma unroll
    for (int nr = 0; nr < NR; ++nr)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
            s_red[wave][nr * MG + mg][lane] = acc[nr][mg];
    __syncthreads();

    Epilogue ep{g.D, g.C, g.alpha, g.beta, g.M, g.N, g.ldd, g.ldc, g.d_vec, g.c_vec, g.c_f32};
    constexpr int FPW = (NF + 3) / 4;  // blocks per wave
    v4f sum[FPW];
#pragma unroll
    for (int i = 0; i < FPW; ++i) {
        const int f = i * 4 + wave;
        if (f < NF)
            sum[i] = ((s_red[0][f][lane] + s_red[1][f][lane]) + s_red[2][f][lane]) + s_red[3][f][lane];
    }
    auto block_mn = [&](int f, int &m, int &n) {
        const int nr = f / MG, mg = f - nr * MG;
        m = mg * 16 + (lane & 15);
        n = n0 + nr * 16 + 4 * (lane >> 4);
    };
    if (g.split == 1) {
#pragma unroll
        for (int i = 0; i < FPW; ++i) {
            const int f = i * 4 + wave;
            if (f < NF) {
                int m, n;
                block_mn(f, m, n);
                store_quad(ep, m, n, sum[i]);
            }
        }
        return;
    }
    // fp32 partials of this chunk: [tile][z][block][lane] float4s
    constexpr uint32_t PART = NF * 64 * 16;  // bytes per workgroup partial
    const auto rws = make_rsrc_u(g.ws + (size_t)t * g.split * (PART / 4), (uint32_t)(g.split * PART));
#pragma unroll
    for (int i = 0; i < FPW; ++i) {
        const int f = i * 4 + wave;
        if (f < NF)
            store16_coherent(rws, z * PART + (uint32_t)((f * 64 + lane) * 16), sum[i]);
    }
    if (!split_arrive_last(g.counters + t, g.split))
        return;
#pragma unroll
    for (int i = 0; i < FPW; ++i) {
        const int f = i * 4 + wave;
        if (f < NF) {
            const uint32_t idx = (uint32_t)((f * 64 + lane) * 16);
            // four chunks in flight at a time, added in z order (a chunk
            // past the split reads zeros from past the range and is not added)
            v4f tot = load16_coherent(rws, idx);
            for (int zz = 1; zz < g.split; zz += 4) {
                v4f part[4];
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    part[h] = load16_coherent(rws, zz + h < g.split ? (zz + h) * PART + idx : kOOB);
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    if (zz + h < g.split)
                        tot += part[h];
            }
            int m, n;
            block_mn(f, m, n);
            store_quad(ep, m, n, tot);
        }
    }
}

template <int MG, int NR, bool BPACK, bool APACK>
static void launch_skinny(const GemmArgs &g, int grid, hipStream_t s)
{
    // 16-byte scale groups need 16-aligned scale rows and whole 16-block
    // groups (with both scale operands packed no row-major group is read)
    if constexpr (APACK) {
        hipLaunchKernelGGL((mx_skinny_kernel<MG, NR, BPACK, false, true, false>), dim3(grid), dim3(256), 0, s, g);
    } else {
        if constexpr (MG == 1) {
            if (g.M == 1) {
                if (g.scale16 || BPACK)  // row-major B scales (if any) in 16-byte groups
                    hipLaunchKernelGGL((mx_skinny_kernel<1, NR, BPACK, true, false, true>), dim3(grid), dim3(256), 0, s, g);
                else
                    hipLaunchKernelGGL((mx_skinny_kernel<1, NR, BPACK, false, false, true>), dim3(grid), dim3(256), 0, s, g);
                return;
            }
        }
        if (g.scale16)
            hipLaunchKernelGGL((mx_skinny_kernel<MG, NR, BPACK, true, false, false>), dim3(grid), dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((mx_skinny_kernel<MG, NR, BPACK, false, false, false>), dim3(grid), dim3(256), 0, s, g);
    }
}

// Wider A formats: one row group (M <= 16 per launch), row-major A scales.
template <int AFMT, bool BPACK>
static void launch_skinny_fmt(const GemmArgs &g, int grid, hipStream_t s)
{
    if (g.M == 1) {
        if (g.scale16 || BPACK)
            hipLaunchKernelGGL((mx_skinny_kernel<1, 1, BPACK, true, false, true, AFMT>), dim3(grid), dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((mx_skinny_kernel<1, 1, BPACK, false, false, true, AFMT>), dim3(grid), dim3(256), 0, s, g);
        return;
    }
    if (g.scale16)
        hipLaunchKernelGGL((mx_skinny_kernel<1, 1, BPACK, true, false, false, AFMT>), dim3(grid), dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL((mx_skinny_kernel<1, 1, BPACK, false, false, false, AFMT>), dim3(grid), dim3(256), 0, s, g);
}

template <int NR, bool BPACK>
static void launch_skinny_bf16a_nr(const GemmArgs &g, int grid, hipStream_t s)
{
    if (g.scale16 || BPACK)
        hipLaunchKernelGGL((mx_skinny_kernel<1, NR, BPACK, true, false, true, kBf16A>), dim3(grid), dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL((mx_skinny_kernel<1, NR, BPACK, false, false, true, kBf16A>), dim3(grid), dim3(256), 0, s, g);
}

void launch_skinny_bf16a(int nr, bool b_packed, const GemmArgs &g, int grid, hipStream_t s)
{
    switch ((nr == 1 ? 0 : nr == 2 ? 1 : 2) * 2 + (b_packed ? 1 : 0)) {
    case 0: launch_skinny_bf16a_nr<1, false>(g, grid, s); break;
    case 1: launch_skinny_bf16a_nr<1, true>(g, grid, s); break;
    case 2: launch_skinny_bf16a_nr<2, false>(g, grid, s); break;
    case 3: launch_skinny_bf16a_nr<2, true>(g, grid, s); break;
    case 4: launch_skinny_bf16a_nr<4, false>(g, grid, s); break;
    default: launch_skinny_bf16a_nr<4, true>(g, grid, s); break;
    }
}

void launch_skinny_wide(int a_fmt, bool b_packed, const GemmArgs &g, int grid, hipStream_t s)
{
    switch (a_fmt * 2 + (b_packed ? 1 : 0)) {
    case 2: launch_skinny_fmt<1, false>(g, grid, s); break;
    case 3: launch_skinny_fmt<1, true>(g, grid, s); break;
    case 4: launch_skinny_fmt<2, false>(g, grid, s); break;
    case 5: launch_skinny_fmt<2, true>(g, grid, s); break;
    case 6: launch_skinny_fmt<3, false>(g, grid, s); break;
    case 7: launch_skinny_fmt<3, true>(g, grid, s); break;
    case 8: launch_skinny_fmt<4, false>(g, grid, s); break;
    case 9: launch_skinny_fmt<4, true>(g, grid, s); break;
    default: break;
    }
}

#define MX_SKINNY(MG, NR)                                                                           \
    {MG, NR, launch_skinny<MG, NR, false, false>, launch_skinny<MG, NR, true, false>,                 \
     launch_skinny<MG, NR, true, true>, "skinny_m" #MG "x16_n" #NR "x16"}
const SkinnyKernel *skinny_kernels(int *count)
{
    static const SkinnyKernel table[] = {
        MX_SKINNY(1, 1), MX_SKINNY(1, 2), MX_SKINNY(1, 4),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}
#undef MX_SKINNY

// ---------------------------------------------------------------------------
// B pre-shuffle.  One thread per 16-byte output chunk: output chunk
// ((n16 * KS + ks) * 64 + lane) holds row n16*16 + lane%16, K-block
// ks*4 + lane/16 (zero outside B).  Scale words: one thread per 32-bit word
// of 32-row group d0 and 8-block group d3; byte d4*2 + d1 of word
// d5*16 + d2 is scale[d0*32 + d1*16 + d2][d3*8 + d4*4 + d5] (0x7F outside).

__global__ void __launch_bounds__(256) mx_pack_b_kernel(uint8_t *Bp, const uint8_t *B, int N, int KB,
                                                        int64_t ldb_b, int KS, int64_t total)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total)
        return;
    const int lane = (int)(idx & 63);
    const int64_t q = idx >> 6;
    const int ks = (int)(q % KS);
    const int64_t n16 = q / KS;
    const int64_t row = n16 * 16 + (lane & 15);
    const int kb = ks * 4 + (lane >> 4);
    v4i v = {0, 0, 0, 0};
    if (row < N && kb < KB)
        v = *reinterpret_cast<const v4i *>(B + row * ldb_b + (int64_t)kb * 16);
    *reinterpret_cast<v4i *>(Bp + idx * 16) = v;
}

__global__ void __launch_bounds__(256) mx_pack_sb_kernel(uint32_t *SBp, const uint8_t *SB, int N, int KB,
                                                         int64_t ldsb, int sn8, int64_t total)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total)
        return;
    const int lane = (int)(idx & 63);
    const int64_t q = idx >> 6;
    const int d3 = (int)(q % sn8);
    const int64_t d0 = q / sn8;
    const int d5 = lane >> 4, d2 = lane & 15;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int d4 = j >> 1, d1 = j & 1;
        const int64_t row = d0 * 32 + d1 * 16 + d2;
        const int col = d3 * 8 + d4 * 4 + d5;
        const uint32_t b = (row < N && col < KB) ? SB[row * ldsb + col] : 0x7Fu;
        w |= b << (8 * j);
    }
    SBp[idx] = w;
}

void launch_pack_b(uint8_t *Bp, const uint8_t *B, int N, int KB, int64_t ldb_b, hipStream_t s)
{
    const int KS = (KB + 3) / 4;
    const int64_t total = (int64_t)((N + 15) / 16) * KS * 64;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(mx_pack_b_kernel, dim3((unsigned)blocks), dim3(256), 0, s, Bp, B, N, KB, ldb_b, KS, total);
}

__global__ void __launch_bounds__(256) mx_zero_words_kernel(uint32_t *p, int64_t words)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < words)
        p[i] = 0u;
}

void launch_zero_words(uint32_t *p, size_t words, hipStream_t s)
{
    const int64_t blocks = ((int64_t)words + 255) / 256;
    hipLaunchKernelGGL(mx_zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, (int64_t)words);
}

void launch_pack_sb(uint32_t *SBp, const uint8_t *SB, int N, int KB, int64_t ldsb, hipStream_t s)
{
    const int sn8 = (KB + 7) / 8;
    const int64_t total = (int64_t)((N + 31) / 32) * sn8 * 64;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(mx_pack_sb_kernel, dim3((unsigned)blocks), dim3(256), 0, s, SBp, SB, N, KB, ldsb, sn8,
                       total);
}

}  // namespace mx

// Tiled MXFP4 GEMM kernel for gfx950: each workgroup of 4 or 8 wave64s
// (WM x WN waves, each owning a TM x TN sub-tile) computes a BM x BN tile of
// D over one K chunk.
//
// Data movement per 256-K stage:
//   - operand tiles go from HBM/L2 straight into LDS with 16-byte-per-lane
//     buffer loads (no VGPR round trip), double-buffered;
//   - LDS holds each operand as lane-linear 1 KiB chunks (16 rows x 128 K,
//     one instruction operand each), so every fragment read is one
//     conflict-free 16-byte ds_read per lane at chunk + 16*lane;
//   - scales are staged through registers into LDS words that already hold
//     the four bytes one lane needs for two 16-row groups x two 128-K steps
//     (the word layout of the asm_f4gemm README's scale shuffle, "Data
//     layouts"), so one 4-byte LDS read feeds four matrix instructions and
//     op_sel picks the byte (the dense FP6 tile keeps those words in
//     registers).
// Out-of-range rows and K blocks are zero-filled by the buffer loads'
// range check, so no caller padding is needed.
//
// Split K: workgroup (tile, z) reduces K-blocks [z*kb_per_split, ...).  With
// more than one chunk every workgroup stores its fp32 partial tile; the last
// one to arrive adds the partials in the fixed order z = 0, 1, ... and runs
// the epilogue, so results do not depend on arrival order.
#include "mx_args.hpp"
#include "mx_device.hpp"
#include "mx_pipe.hpp"

#include <type_traits>

namespace mx {

// s_waitcnt with vmcnt(0) only (expcnt and lgkmcnt left at their maxima):
// waits for this wave's outstanding memory loads, including LDS-direct ones.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Scale bytes of one stage for one 32-row group, as loaded: rows r0 and
// r0+16, 8 K-blocks each (word 0 = blocks 0..3, word 1 = blocks 4..7).
struct ScaleRows {
    v2u r0, r1;
};

// Loads the two rows' 8 stage scale bytes.  SVEC: one 8-byte load per row
// (K-block count and row pitch multiples of 8, so a stage is never partly
// outside the chunk).  Otherwise byte loads, blocks at or past kb_end read
// from an out-of-range offset (zero).  `own` false turns every load into an
// out-of-range one; nothing branches.
template <bool SVEC>
__device__ __forceinline__ ScaleRows load_scale_rows(__amdgpu_buffer_rsrc_t r, int64_t ld, int row0,
                                                     int kb_s, int kb_end, bool own)
{
    ScaleRows s;
    const uint32_t o0 = own ? (uint32_t)(row0 * ld + kb_s) : kOOB;
    const uint32_t o1 = own ? (uint32_t)((row0 + 16) * ld + kb_s) : kOOB;
    if constexpr (SVEC) {
        s.r0 = load8(r, o0);
        s.r1 = load8(r, o1);
    } else {
        uint32_t b0[2] = {0, 0}, b1[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool ok = kb_s + j < kb_end;
            b0[j >> 2] |= load1(r, ok ? o0 + j : kOOB) << (8 * (j & 3));
            b1[j >> 2] |= load1(r, ok ? o1 + j : kOOB) << (8 * (j & 3));
        }
        s.r0 = v2u{b0[0], b0[1]};
        s.r1 = v2u{b1[0], b1[1]};
    }
    return s;
}

// Word for lane (K-block d5 of the step, row d2): bytes
// [step0 row r0, step0 row r0+16, step1 row r0, step1 row r0+16].
__device__ __forceinline__ uint32_t scale_word(const ScaleRows &s, int d5)
{
    const int sh = 8 * d5;
    return ((s.r0[0] >> sh) & 0xFFu) | (((s.r1[0] >> sh) & 0xFFu) << 8) |
           (((s.r0[1] >> sh) & 0xFFu) << 16) | (((s.r1[1] >> sh) & 0xFFu) << 24);
}

// Whole-tile form of the staged epilogue (every row and column inside D,
// beta == 0): D[m_base + r][n_base + c] = bf16(alpha * acc), staged through
// the wave's private LDS region exactly as store_tile_staged does, without
// the bounds checks.  `lane` comes in through an opaque register so that the
// persistent kernel recomputes the addresses per tile instead of hoisting
// them out of its tile loop (where they would be spilled, and every reload
// would wait for all outstanding memory operations).
template <int FM, int FN>
__device__ __forceinline__ void store_whole_tile_staged(uint16_t *D, int64_t ldd, float alpha, int m_base,
                                                        int n_base, const v4f (&acc)[FN][FM], uint8_t *lds,
                                                        int lane)
{
    constexpr int RB = FN * 32;  // bytes per row of the wave tile
    constexpr int CH = RB / 16;  // 16-byte chunks per row
    constexpr int RPI = 64 / CH; // rows per copy-out instruction
    static_assert(CH == 2 || CH == 4 || CH == 8 || CH == 16, "row chunking");
    // (the swizzle of store_tile_staged)
    auto sw = [](int r) { return CH == 16 ? (r & 15) : ((r >> 1) & (CH - 1)); };
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int r = fm * 16 + (lane & 15);
            const int j = fn * 2 + (lane >> 5);
            v2u o;
            o[0] = bf16x2_rne(alpha * acc[fn][fm][0], alpha * acc[fn][fm][1]);
            o[1] = bf16x2_rne(alpha * acc[fn][fm][2], alpha * acc[fn][fm][3]);
            *reinterpret_cast<v2u *>(lds + r * RB + ((j ^ sw(r)) * 16) + ((lane >> 4) & 1) * 8) = o;
        }
    const int r0 = lane / CH, c = lane & (CH - 1);
    uint16_t *d0 = D + (int64_t)(m_base + r0) * ldd + n_base + c * 8;
#pragma unroll
    for (int i = 0; i < FM * 16 / RPI; ++i) {
        const int r = i * RPI + r0;
        const v4i v = *reinterpret_cast<const v4i *>(lds + r * RB + ((c ^ sw(r)) * 16));
        __builtin_nontemporal_store(v, reinterpret_cast<v4i *>(d0 + (int64_t)(i * RPI) * ldd));
    }
}

// AFMT: A's format (0 FP4; 1 FP8 E4M3 or 2 BF8 E5M2; 3 FP6 E2M3 or 4 FP6
// E3M2 in the padded layout of mx_fp6.hip; B is FP4).  An 8-bit A row holds
// 256 bytes per 256-K stage: the stage is two FP4-shaped A tiles, one per
// 128-K step (rows of 128 bytes, the same swizzle), and a lane's operand for
// step ks is chunks g and g+4 of that step's tile -- the two 16-element runs
// K 16g.. and 64+16g.. the 8-bit instruction reads.  A padded FP6 row has the
// same shape, with K-block g's 24 bytes in those two chunks (the first 8
// bytes of chunk g+4), so the same reads feed the FP6 instruction.
// A6D (FP6 A in the dense operand order of mx_fp6.hip, 256 x 256, packed B
// and scales): a stage of A is 3 KiB per 16-row group, the lanes' 24-byte
// operands back to back, read as three 8-byte pieces per lane; A and B fill
// the LDS, so each wave loads its scale words into registers.
// PERSIST (a tile with one workgroup per CU; launched for 256 x 256 with
// packed B and A scales, FP4 or dense FP6): one workgroup per CU walks its tiles in the order
// the plain grid runs them (hardware id blockIdx + i * grid, through the same
// XCD remap).  After a tile's last stage (which reads buffer 1) it issues the
// next tile's first stage into buffer 0, then writes D through buffer 1's A
// half, 1/PARTS of the wave tile per pass: the next tile's load latency
// hides behind the epilogue, and the epilogue's stores drain behind the next
// tile's first stage.  Needs split 1, beta == 0 with the staged epilogue, an
// even stage count and M, N multiples of the tile, so that every wave issues
// exactly STORES stores after those loads (the host checks).
//
// BLAY: B's storage.  0: codes [N][K] and scales [N][KB], row-major; 1: both
// as mxgemm_pack_b writes them; 2: codes MN-major [K][N] (row k holds the N
// columns at that k), scales row-major; 3: MN-major codes, scales shuffled
// as mxgemm_pack_b shuffles them.  An MN-major stage is 256 K-rows of BN/2
// bytes in LDS; a B fragment (16 columns x 128 K) is two transposed reads
// ("CDNA4 MFMA transpose load builtins", ds_read_tr4_b64: each 16-lane group
// names 16 K-rows of 8 bytes, i.e. 16 columns, and every lane receives its
// own column's 16 K values as 8 bytes, row q in nibble q; the table of that
// page's "Hardware constraints" splits the K positions over the two calls),
// K-rows 32g .. 32g+15 and 32g+16 .. 32g+31 of the step for lane group g,
// which is the K-block g the instruction reads from lane group g.
template <int BM, int BN, int WM, int WN, int BLAY, bool SVEC, bool SAPACK, int AFMT = 0, bool PERSIST = false,
          bool A6D = false>
__global__ void __launch_bounds__(64 * WM * WN) mx_tile_kernel(GemmArgs g)
{
    static_assert(AFMT == 0 || (AFMT >= 1 && AFMT <= 4 && (!SAPACK || A6D)),
                  "8-bit or padded FP6 A with row-major A scales, or dense FP6 A");
    static_assert(!A6D || (AFMT >= 3 && BLAY == 1 && SAPACK), "dense FP6 A with packed B and scales");
    static_assert(BLAY >= 0 && BLAY <= 3 && (AFMT == 0 || BLAY <= 1), "B layouts");
    constexpr bool BPACK = BLAY == 1;                 // packed codes
    constexpr bool BKN = BLAY >= 2;                   // MN-major codes
    constexpr bool SBPACK = BLAY == 1 || BLAY == 3;   // packed B scales
    static_assert(!SAPACK || SBPACK, "packed A scales come with packed B scales");
    // MN-major stage geometry: bytes per K-row, 16-byte chunks per K-row,
    // K-rows per direct-to-LDS instruction and per 256-byte bank window.
    // Chunk c of K-row r sits at slot c ^ ((r / KN_RPW) % KN_CPR): the 16
    // K-rows one lane group names in a transposed read then fall on 16
    // different 8-byte bank positions.
    constexpr int KN_ROWB = BN / 2, KN_CPR = BN / 32;
    constexpr int KN_RPI = 1024 / KN_ROWB, KN_RPW = 256 / KN_ROWB;
    constexpr int AREG = AFMT == 0 ? 1 : 2;  // FP4-shaped A tiles per stage
    constexpr int NW = WM * WN;                // waves per workgroup
    constexpr int NT = 64 * NW;                // threads per workgroup
    constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
    constexpr int FM = TM / 16, FN = TN / 16;  // 16-row fragments per wave
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    static_assert(FM % 2 == 0 && FN % 2 == 0, "scale words cover 32-row groups");
    // bytes per stage (dense FP6 A: 16-row groups of two 1536-byte steps)
    constexpr int A_STAGE = A6D ? BM * 192 : BM * 128 * AREG, B_STAGE = BN * 128;
    constexpr int A_CH = A_STAGE / 1024, B_CH = BN / 8;  // 1 KiB chunks per stage
    static_assert(A_CH % NW == 0 && B_CH % NW == 0, "chunks split evenly over waves");
    constexpr int SA_W = BM / 32 * 64, SB_W = BN / 32 * 64;  // scale words per stage
    constexpr int SC_W = SA_W + SB_W + 64;                   // + a scratch row for idle threads
    constexpr int SBP_PER_THREAD = (SB_W + NT - 1) / NT;     // packed-scale words per thread
    constexpr int SAP_PER_THREAD = (SA_W + NT - 1) / NT;
    static_assert(BM / 2 + BN / 2 <= NT, "one scale row pair per thread");

    // The two halves of each double buffer are distinct LDS objects and every
    // access names one of them at compile time: the compiler can then tell
    // the next stage's direct-to-LDS loads from this stage's fragment reads
    // and does not make the reads wait for the loads.
    __shared__ __attribute__((aligned(1024))) uint8_t s_a0[A_STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t s_a1[A_STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t s_b0[B_STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t s_b1[B_STAGE];
    // [SA words | SB words | scratch]; the dense FP6 tile's operands fill
    // the LDS, and its waves load their scale words into registers instead
    __shared__ uint32_t s_sc0[A6D ? 1 : SC_W];
    __shared__ uint32_t s_sc1[A6D ? 1 : SC_W];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS/chunk math scalar
    const int wave_m = wave % WM, wave_n = wave / WM;

    // ---- which tile and K chunk, and the operand sources rebased at the
    // tile (offsets stay below 2^31).  Per stage the base advances by the
    // stage's K offset and the range shrinks by the same amount, so a lane's
    // offset inside a stage is its fixed lane part plus a wave-uniform chunk
    // part.  A stage that must not load gets an empty range: every load
    // returns zero without traffic.
    const int tiles = g.tiles_m * g.tiles_n;
    int z, t, m0, n0, kb_begin, kb_end, nst;
    // MN-major B: this lane's byte offset inside a stage's K-rows for every
    // load instruction of the wave (instruction c adds c * KN_RPI K-rows),
    // or an offset past any range (2^31) for chunks beyond column N.  Lane
    // l fills slot l % KN_CPR of K-row c * KN_RPI + l / KN_CPR, i.e. chunk
    // slot ^ ((4c + (l / KN_CPR) / KN_RPW) % KN_CPR), and 4c % KN_CPR depends
    // on c only through c % 2 = wave % 2 (c = i * NW + wave, NW even).
    uint32_t kn_lane = 0;
    static_assert(NW % 2 == 0 && KN_RPI == 4 * KN_RPW, "MN-major load geometry");
    const uint8_t *a_base, *b_base;
    uint32_t a_bytes, b_bytes;
    __amdgpu_buffer_rsrc_t rsa, rsb;
    // Row-major operands move in whole 128-byte lines: one load instruction
    // covers 8 rows x the stage's 128 bytes (lane l: row l/8 of the h-th
    // 8-row half of a 16-row group, 16-byte chunk (l%8) ^ sw(row)).  The
    // resulting LDS layout of a 16-row group (2 KiB) puts row r, chunk c at
    // 16-byte slot (r/8)*64 + (r%8)*8 + (c ^ sw(r)), sw(r) = 2*bit1(r) +
    // 4*bit3(r).  A 16-byte LDS read serves 16 lanes per cycle: lanes 0-31
    // and 32-63 separately, each split by the parity of lane bits 2-4
    // (measured on gfx950 with two-lane bank probes).  Under that grouping a
    // fragment read (row lane%16, chunk 4ks + lane/16) touches 16 distinct
    // 16-byte bank slots, i.e. all 64 banks once; the earlier swizzle
    // c ^ (r%8) ^ (r/8), laid out for lanes 0-15 per cycle, doubled every
    // fragment read (measured 2-way with the LDS conflict counters).
    const int kc_lane = (lane & 7) ^ (2 * ((lane >> 4) & 1));  // chunk of lane l in a half-0 load
    const uint32_t a_lane = (uint32_t)((lane >> 3) * g.lda_b + kc_lane * 16);
    uint32_t b_lane, b_rg_stride;
    if constexpr (BPACK) {
        b_lane = (uint32_t)(lane * 16);
        b_rg_stride = (uint32_t)(g.ks_total * 1024);
    } else {
        b_lane = (uint32_t)((lane >> 3) * g.ldb_b + kc_lane * 16);
        b_rg_stride = (uint32_t)(16 * g.ldb_b);
    }
    auto load_src = [&](int lg) __attribute__((always_inline)) {
        z = lg / tiles;
        t = lg - z * tiles;
        const int per_group = g.group_m * g.tiles_n;
        const int grp = t / per_group;
        const int first_m = grp * g.group_m;
        const int gsz = min(g.tiles_m - first_m, g.group_m);
        const int within = t - grp * per_group;
        const int tm = first_m + within % gsz;
        const int tn = within / gsz;
        m0 = tm * BM;
        n0 = tn * BN;
        kb_begin = z * g.kb_per_split;
        kb_end = min(g.KB, kb_begin + g.kb_per_split);
        nst = (kb_end - kb_begin + 7) >> 3;
        // (every range below is under 2^31 bytes: the host rejects strides
        // and K for which a 256-row tile's would not be)
        const int rows_a = min(BM, g.M - m0);
        if constexpr (A6D) {
            // lda_b: bytes per 16-row group
            const int grp16 = min(BM / 16, (g.M + 15) / 16 - m0 / 16);
            a_base = g.A + (int64_t)(m0 / 16) * g.lda_b;
            a_bytes = (uint32_t)((int64_t)grp16 * g.lda_b);
        } else {
            a_base = g.A + (int64_t)m0 * g.lda_b;
            a_bytes = (uint32_t)((int64_t)rows_a * g.lda_b);
        }
        if constexpr (SAPACK) {
            const int m32 = m0 / 32, grp32 = min(BM / 32, (g.M + 31) / 32 - m32);
            rsa = make_rsrc(g.SA + (int64_t)m32 * g.sn8 * 256, (uint32_t)((int64_t)grp32 * g.sn8 * 256));
        } else {
            rsa = make_rsrc(g.SA + (int64_t)m0 * g.ldsa, (uint32_t)((int64_t)rows_a * g.ldsa));
        }
        if constexpr (BPACK) {
            const int n16 = n0 / 16, grp16 = min(BN / 16, (g.N + 15) / 16 - n16);
            b_base = g.B + (int64_t)n16 * g.ks_total * 1024;
            b_bytes = (uint32_t)((int64_t)grp16 * g.ks_total * 1024);
        } else if constexpr (BKN) {
            b_base = g.B;  // each stage rebases at its first K-row
            b_bytes = 0;
            const int chunk = (lane % KN_CPR) ^ ((4 * wave + (lane / KN_CPR) / KN_RPW) % KN_CPR);
            kn_lane = n0 + 32 * chunk < g.N ? (uint32_t)((lane / KN_CPR) * g.ldb_b + n0 / 2 + 16 * chunk)
                                            : 0x80000000u;
        } else {
            const int rows_b = min(BN, g.N - n0);
            b_base = g.B + (int64_t)n0 * g.ldb_b;
            b_bytes = (uint32_t)((int64_t)rows_b * g.ldb_b);
        }
        if constexpr (SBPACK) {
            const int n32 = n0 / 32, grp32 = min(BN / 32, (g.N + 31) / 32 - n32);
            rsb = make_rsrc(g.SB + (int64_t)n32 * g.sn8 * 256, (uint32_t)((int64_t)grp32 * g.sn8 * 256));
        } else {
            const int rows_b = min(BN, g.N - n0);
            rsb = make_rsrc(g.SB + (int64_t)n0 * g.ldsb, (uint32_t)((int64_t)rows_b * g.ldsb));
        }
    };
    // units of work are (tile, K chunk) pairs: the plain grid runs one per
    // workgroup, the persistent one walks hardware ids blockIdx + i * grid
    const int units = tiles * g.split;
    int unit_hw = blockIdx.x;
    load_src(xcd_remap(unit_hw, PERSIST ? units : (int)gridDim.x));

    // ---- stage loaders
    auto issue_operands = [&](int kt, bool on, auto bufc) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        uint8_t *dst_a = BUF ? s_a1 : s_a0;
        uint8_t *dst_b = BUF ? s_b1 : s_b0;
        const int kb_s = kb_begin + kt * 8;
        // K offset of the stage: bytes along a row (row-major), 1 KiB steps
        // (packed B) or 1536-byte steps (dense FP6 A)
        const uint32_t a_k = A6D ? (uint32_t)(kb_s >> 2) * 1536 : (uint32_t)kb_s * 16 * AREG;
        const uint32_t b_k = BPACK ? (uint32_t)(kb_s >> 2) * 1024 : (uint32_t)kb_s * 16;
        const auto ra = make_rsrc(a_base + a_k, on ? a_bytes - a_k : 0u);
        // MN-major: the stage's K-rows kb_s*32 .. up to the chunk end; rows
        // past it are outside the range and load zeros
        const auto rb = BKN ? make_rsrc_u(b_base + (int64_t)kb_s * 32 * g.ldb_b,
                                          on ? (uint32_t)(min(256, (kb_end - kb_s) * 32) * g.ldb_b) : 0u)
                            : make_rsrc(b_base + b_k, on ? b_bytes - b_k : 0u);
        // chunk (K-block of the stage) a row-major lane loads in half h
        const int kc0 = kc_lane, kc1 = kc0 ^ 4;
        // dense FP6: the lane's byte offset, opaque per stage, so that the
        // compiler forms each load's offset when it issues it instead of
        // keeping ten loop-invariant offsets live (which spilled them)
        uint32_t lane16 = (uint32_t)lane * 16;
        if constexpr (A6D)
            asm volatile("" : "+v"(lane16));
#pragma unroll
        for (int i = 0; i < A_CH / NW; ++i) {
            const int c = i * NW + wave;
            if constexpr (A6D) {
                // dense FP6: 1 KiB piece c % 3 of 16-row group c / 3's 3 KiB
                // stage (zeros past M and K are in the copy itself)
                load16_to_lds(ra, (lds_void *)(dst_a + c * 1024),
                              (uint32_t)((c / 3) * g.lda_b) + (uint32_t)((c % 3) * 1024) + lane16);
                continue;
            }
            const int reg = AREG == 1 ? 0 : c / (BM / 8), cc = AREG == 1 ? c : c % (BM / 8);  // A tile, chunk
            const int rows8 = cc * 8, h = cc & 1;            // 8-row half h of group cc/2
            uint32_t off = a_lane + (uint32_t)(rows8 * g.lda_b) + (h ? (uint32_t)((kc1 - kc0) * 16) : 0u);
            if constexpr (AREG > 1)
                off += (uint32_t)(reg * 128);
            if constexpr (!SVEC) {  // K tail: blocks at or past the chunk end read as zero
                // (the K-block chunk kc of the step's tile holds: 8-bit A
                // chunk kc covers block kc / 2, padded FP6 block kc % 4)
                const int kc = h ? kc1 : kc0;
                off = kb_s + (AREG == 1 ? kc : 4 * reg + (AFMT >= 3 ? kc & 3 : kc / 2)) < kb_end ? off : kOOB;
            }
            load16_to_lds(ra, (lds_void *)(dst_a + c * 1024), off);
        }
#pragma unroll
        for (int i = 0; i < B_CH / NW; ++i) {
            const int c = i * NW + wave;
            uint32_t off;
            if constexpr (BPACK) {
                // packed B: 1 KiB instruction operands, contiguous
                const int rg = c >> 1, ks = c & 1;
                off = (A6D ? lane16 : b_lane) + (uint32_t)rg * b_rg_stride + (uint32_t)(ks * 1024);
            } else if constexpr (BKN) {
                // MN-major: instruction c fills K-rows c * KN_RPI .. (a range
                // below 2^31 - 2^31 + this, so past-N lanes stay out of range)
                off = kn_lane + (uint32_t)(c * KN_RPI) * (uint32_t)g.ldb_b;
            } else {
                const int rows8 = c * 8, h = c & 1;
                off = b_lane + (uint32_t)(rows8 * g.ldb_b) + (h ? (uint32_t)((kc1 - kc0) * 16) : 0u);
                if constexpr (!SVEC)
                    off = kb_s + (h ? kc1 : kc0) < kb_end ? off : kOOB;
            }
            load16_to_lds(rb, (lds_void *)(dst_b + c * 1024), off);
        }
    };

    // scale-row ownership: thread < BM/2 owns A row pair tid; the next BN/2
    // threads own B row pairs (row-major B scales only)
    const bool own_a = !SAPACK && tid < BM / 2;
    const int ua = own_a ? tid : 0;
    const bool own_b = !SBPACK && tid >= BM / 2 && tid < BM / 2 + BN / 2;
    const int ub = own_b ? tid - BM / 2 : 0;
    // LDS word index (per d5 add 16*d5) each thread commits its A / B words to
    const int wa = own_a ? (ua >> 4) * 64 + (ua & 15) : SA_W + SB_W + lane;
    const int wb = own_b ? SA_W + (ub >> 4) * 64 + (ub & 15) : SA_W + SB_W + lane;

    ScaleRows sa_rows, sb_rows;
    uint32_t sbp[SBP_PER_THREAD], sap[SAP_PER_THREAD];
    // dense FP6: this wave's packed scale words of a stage (its 32-row groups
    // of A and of B), one register set per buffer
    uint32_t rsaw[2][FM / 2], rsbw[2][FN / 2];
    auto issue_scales = [&](int kt, bool on, auto bufc) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        const int kb_s = kb_begin + kt * 8;
        if constexpr (A6D) {
            // (past the last stage these read the next chunk's words or, past
            // the scale rows, zeros from the range check: never used)
#pragma unroll
            for (int p = 0; p < FM / 2; ++p)
                rsaw[BUF][p] = load4(rsa, (uint32_t)((((wave_m * (FM / 2) + p) * g.sn8 + (kb_s >> 3)) * 64 + lane) * 4));
#pragma unroll
            for (int p = 0; p < FN / 2; ++p)
                rsbw[BUF][p] = load4(rsb, (uint32_t)((((wave_n * (FN / 2) + p) * g.sn8 + (kb_s >> 3)) * 64 + lane) * 4));
            return;
        }
        if constexpr (SAPACK) {
            // packed words are already the LDS words: word q of the stage is
            // word q & 63 of 32-row group q / 64's chunk for this 8-block step
#pragma unroll
            for (int i = 0; i < SAP_PER_THREAD; ++i) {
                const int q = i * NT + tid;
                const uint32_t off = on && q < SA_W
                                         ? (uint32_t)((((q >> 6) * g.sn8 + (kb_s >> 3)) * 64 + (q & 63)) * 4)
                                         : kOOB;
                sap[i] = load4(rsa, off);
            }
        } else {
            sa_rows = load_scale_rows<SVEC>(rsa, g.ldsa, (ua >> 4) * 32 + (ua & 15), kb_s, kb_end, on && own_a);
        }
        if constexpr (SBPACK) {
#pragma unroll
            for (int i = 0; i < SBP_PER_THREAD; ++i) {
                const int q = i * NT + tid;
                const uint32_t off = on && q < SB_W
                                         ? (uint32_t)((((q >> 6) * g.sn8 + (kb_s >> 3)) * 64 + (q & 63)) * 4)
                                         : kOOB;
                sbp[i] = load4(rsb, off);
            }
        } else {
            sb_rows = load_scale_rows<SVEC>(rsb, g.ldsb, (ub >> 4) * 32 + (ub & 15), kb_s, kb_end, on && own_b);
        }
    };
    auto commit_scales = [&](auto bufc) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        if constexpr (A6D)
            return;
        uint32_t *dsc = BUF ? s_sc1 : s_sc0;
        if constexpr (SAPACK) {
#pragma unroll
            for (int i = 0; i < SAP_PER_THREAD; ++i) {
                const int q = i * NT + tid;
                dsc[q < SA_W ? q : SA_W + SB_W + lane] = sap[i];
            }
        } else {
#pragma unroll
            for (int d5 = 0; d5 < 4; ++d5)
                dsc[wa + (own_a ? 16 * d5 : 0)] = scale_word(sa_rows, d5);
        }
        if constexpr (SBPACK) {
#pragma unroll
            for (int i = 0; i < SBP_PER_THREAD; ++i) {
                const int q = i * NT + tid;
                dsc[q < SB_W ? SA_W + q : SA_W + SB_W + lane] = sbp[i];
            }
        } else {
#pragma unroll
            for (int d5 = 0; d5 < 4; ++d5)
                dsc[wb + (own_b ? 16 * d5 : 0)] = scale_word(sb_rows, d5);
        }
    };

    // LDS byte offset of this lane's 16 bytes of a row-major fragment inside
    // its 16-row group (row lane%16, K-block lane/16 of step 0; step 1 flips
    // chunk bit 2)
    const int fr = lane & 15;
    const int sw_fr = 2 * ((fr >> 1) & 1) + 4 * ((fr >> 3) & 1);
    const uint32_t rl0 = (uint32_t)(((fr >> 3) * 64 + (fr & 7) * 8 + ((lane >> 4) ^ sw_fr)) * 16);
    const uint32_t rl1 = rl0 ^ 64u;
    // MN-major fragment reads: lane (group g, row i) names K-row 32g + i of
    // the step (call 1; call 2 is 16 K-rows further), whose chunks are
    // swizzled by h = (i / KN_RPW) % KN_CPR (the same for both calls and
    // every step: 16, 32 and 128 are multiples of KN_RPW * KN_CPR)
    const uint32_t kn_row = (uint32_t)((lane >> 4) * 32 + fr) * KN_ROWB;
    const int kn_h = (fr / KN_RPW) % KN_CPR;

    // ---- main loop
    // Accumulators get their first value from the first stage's matrix
    // instructions (zero accumulator input), never from a register move, so
    // the register allocator keeps them in the accumulation registers across
    // the loop.
    v4f acc[FN][FM];

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;

    // One stage, one basic block: prefetch stage kt+1 into the other buffer,
    // multiply stage kt, then wait for the prefetch and publish its scales.
    // LOADS_AT places the prefetch: -1 lets the compiler interleave it, P >= 0
    // issues it just before fragment step P (P = ks * FN + fn; 0 = before the
    // first multiply).
    auto stage = [&](int kt, auto bufc, auto firstc, auto loadsc) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        constexpr bool FIRST = decltype(firstc)::value;
        constexpr int LOADS_AT = decltype(loadsc)::value;
        using Next = std::integral_constant<int, BUF ^ 1>;
        const bool more = kt + 1 < nst;
        auto prefetch = [&]() __attribute__((always_inline)) {
            if constexpr (LOADS_AT >= 0)
                __builtin_amdgcn_sched_barrier(0);
            issue_operands(kt + 1, more, Next{});
            issue_scales(kt + 1, more, Next{});
            if constexpr (LOADS_AT >= 0)
                __builtin_amdgcn_sched_barrier(0);
        };
        if constexpr (LOADS_AT <= 0)
            prefetch();
        const uint8_t *sa_tile = BUF ? s_a1 : s_a0;
        const uint8_t *sb_tile = BUF ? s_b1 : s_b0;
        const uint32_t *ssc = BUF ? s_sc1 : s_sc0;
        uint32_t saw[FM / 2], sbw[FN / 2];
#pragma unroll
        for (int p = 0; p < FM / 2; ++p)
            saw[p] = A6D ? rsaw[BUF][p] : ssc[(wave_m * (FM / 2) + p) * 64 + lane];
#pragma unroll
        for (int p = 0; p < FN / 2; ++p)
            sbw[p] = A6D ? rsbw[BUF][p] : ssc[SA_W + (wave_n * (FN / 2) + p) * 64 + lane];
        if constexpr (A6D) {
            // dense FP6, per 128-K step: the four A operands (three 8-byte
            // reads each at a 24-byte lane stride: 32 lanes per cycle on 64
            // distinct banks), then the eight B fragments, each read one
            // fragment ahead of its multiplies.  A scheduling barrier after
            // each fragment's multiplies keeps the compiler from issuing all
            // of a step's reads up front, which spilled.
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                v8i af[FM];
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const uint8_t *t = sa_tile + (wave_m * FM + fm) * 3072 + ks * 1536 + lane * 24;
                    const v2u p0 = *reinterpret_cast<const v2u *>(t);
                    const v2u p1 = *reinterpret_cast<const v2u *>(t + 8);
                    const v2u p2 = *reinterpret_cast<const v2u *>(t + 16);
                    af[fm] = v8i{(int)p0[0], (int)p0[1], (int)p1[0], (int)p1[1], (int)p2[0], (int)p2[1], 0, 0};
                }
                auto read_b = [&](int fn) __attribute__((always_inline)) {
                    return *reinterpret_cast<const v4i *>(sb_tile + ((wave_n * FN + fn) * 2 + ks) * 1024 + lane * 16);
                };
                v4i bq[2];
                bq[0] = read_b(0);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    if constexpr (LOADS_AT > 0) {
                        if (ks * FN + fn == LOADS_AT)
                            prefetch();
                    }
                    if (fn + 1 < FN)
                        bq[(fn + 1) & 1] = read_b(fn + 1);
                    const v4i bf = bq[fn & 1];
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
                        acc[fn][fm] = mma_sel_wide<kFmtHw[AFMT]>(
                            ks * 2 + (fn & 1), ks * 2 + (fm & 1), bf, af[fm],
                            FIRST && ks == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : acc[fn][fm], (int)sbw[fn >> 1],
                            (int)saw[fm >> 1]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            using a_t = typename std::conditional<AFMT == 0, v4i, v8i>::type;
            a_t af[FM];
            const uint32_t rl = ks ? rl1 : rl0;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                if constexpr (AFMT == 0) {
                    af[fm] = *reinterpret_cast<const v4i *>(sa_tile + (wave_m * FM + fm) * 2048 + rl);
                } else {
                    const uint8_t *t = sa_tile + ks * (BM * 128) + (wave_m * FM + fm) * 2048;
                    const v4i lo = *reinterpret_cast<const v4i *>(t + rl0);
                    const v4i hi = *reinterpret_cast<const v4i *>(t + rl1);
                    af[fm] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                if constexpr (LOADS_AT > 0) {
                    if (ks * FN + fn == LOADS_AT)
                        prefetch();
                }
                v4i bf;
                if constexpr (BKN) {
                    // 8-byte unit u of the K-row: columns 16u .. 16u+15 of the tile
                    const int u = wave_n * FN + fn;
                    const uint8_t *t = sb_tile + ks * 128 * KN_ROWB + kn_row + (((u >> 1) ^ kn_h) * 16) + (u & 1) * 8;
                    const v2i lo = lds_tr4(t), hi = lds_tr4(t + 16 * KN_ROWB);
                    bf = v4i{lo[0], lo[1], hi[0], hi[1]};
                } else {
                    const uint32_t bo = BPACK ? ((wave_n * FN + fn) * 2 + ks) * 1024 + lane * 16
                                              : (wave_n * FN + fn) * 2048 + rl;
                    bf = *reinterpret_cast<const v4i *>(sb_tile + bo);
                }
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    if constexpr (AFMT == 0)
                        acc[fn][fm] = mma_sel(ks * 2 + (fn & 1), ks * 2 + (fm & 1), bf, af[fm],
                                              FIRST && ks == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : acc[fn][fm],
                                              (int)sbw[fn >> 1], (int)saw[fm >> 1]);
                    else
                        acc[fn][fm] = mma_sel_wide<kFmtHw[AFMT]>(
                            ks * 2 + (fn & 1), ks * 2 + (fm & 1), bf, af[fm],
                            FIRST && ks == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : acc[fn][fm], (int)sbw[fn >> 1],
                            (int)saw[fm >> 1]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        }
        wait_vmem();
        commit_scales(Next{});
        __syncthreads();
    };

    issue_operands(0, true, B0{});
    issue_scales(0, true, B0{});
    wait_vmem();
    commit_scales(B0{});
    __syncthreads();
    // Stage 0 is peeled (it initialises the accumulators); then pairs of
    // stages keep the buffer choice static, and an odd last stage is peeled
    // so that the loop body has no branch (no join over the accumulators).
    using First = std::true_type;
    using Rest = std::false_type;
    for (;;) {
    auto run = [&](auto loadsc) __attribute__((always_inline)) {
        stage(0, B0{}, First{}, loadsc);
        int kt = 1;
        for (; kt + 2 <= nst; kt += 2) {
            stage(kt, B1{}, Rest{}, loadsc);
            stage(kt + 1, B0{}, Rest{}, loadsc);
        }
        if (kt < nst)
            stage(kt, B1{}, Rest{}, loadsc);
    };
    if constexpr (NW == 8 && SVEC) {
        // Eight waves, two per SIMD (waves w and w + 4).  Each stage's
        // prefetch is 64 direct-to-LDS loads per workgroup, which the CU's
        // load path takes about 16 cycles each to accept; a wave whose load
        // is not yet accepted cannot issue its next multiply either.  Waves
        // 0-3 therefore prefetch before their first multiply and waves 4-7
        // before fragment step 3 (after their first 24 multiplies), so that
        // while one wave of a SIMD waits on the load path the other one
        // multiplies.  8192^3 on one MI355X: issue points (0, 2) were 5 %
        // faster than one common point, and (0, 3) 1.5-2 % faster than
        // (0, 2); (0, 1), (1, 3), (0, 4), (0, 5) and (0, 6) were slower.  The K-tail
        // variant (!SVEC) keeps one issue point: its larger address state
        // spills inside the loop when the loop is instantiated twice.
        // (the dense FP6 tile, eight fragment steps per 128-K step: waves
        // 4-7 at the second step's start, 8192^3 304-305 us against
        // 311-315 us at step 3 and 313-314 us at step 1)
        if (wave >= 4)
            run(std::integral_constant<int, A6D ? 8 : 3>{});
        else
            run(std::integral_constant<int, 0>{});
    } else {
        run(std::integral_constant<int, -1>{});
    }
    if constexpr (PERSIST) {
        const int ep_m0 = m0, ep_n0 = n0;
        const int next_hw = unit_hw + (int)gridDim.x;
        const bool has_next = next_hw < units;
        if (has_next) {
            // the next unit's first stage into the free buffer pair
            // (its last readers passed the barrier ending stage nst - 2)
            load_src(xcd_remap(next_hw, units));
            issue_operands(0, true, B0{});
            issue_scales(0, true, B0{});
        }
        // staged epilogue in the last stage's A buffer: each wave stages
        // 1/PARTS of its tile at a time in a private region of s_a1.  Naming
        // that one array lets the compiler tell the staging accesses from
        // the next stage's direct-to-LDS loads into the other pair, so they
        // do not wait for those loads.
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        constexpr int PARTS = NW * TM * TN * 2 <= A_STAGE ? 1 : NW * TM * TN <= A_STAGE ? 2 : 4;
        constexpr int QREG = (TM / PARTS) * TN * 2;
        static_assert(NW * QREG <= A_STAGE && FM % PARTS == 0, "partial-tile staging fits the A buffer");
        uint8_t *buf = s_a1 + wave * QREG;
#pragma unroll
        for (int part = 0; part < PARTS; ++part) {
            v4f q[FN][FM / PARTS];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int i = 0; i < FM / PARTS; ++i)
                    q[fn][i] = acc[fn][part * (FM / PARTS) + i];
            store_whole_tile_staged<FM / PARTS, FN>(g.D, g.ldd, g.alpha, ep_m0 + wave_m * TM + part * (TM / PARTS),
                                                    ep_n0 + wave_n * TN, q, buf, lane_e);
        }
        if (!has_next)
            return;
        // the first-stage loads were issued before this wave's STORES stores
        // (16-byte stores of 64 / (2 FN) rows each): in-order completion
        // makes them landed at STORES outstanding
        constexpr int STORES = FM * 16 / (64 / (FN * 2));
        wait_vmcnt<STORES>();
        commit_scales(B0{});
        // the stage and its scales are in place, and every wave is done with
        // its staging region before the next stage is loaded over it
        __syncthreads();
        unit_hw = next_hw;
        continue;
    }
    break;
    }

    // ---- epilogue
    Epilogue ep{g.D, g.C, g.alpha, g.beta, g.M, g.N, g.ldd, g.ldc, g.d_vec, g.c_vec, g.c_f32};
    const int mb = m0 + wave_m * TM + (lane & 15);
    const int nb = n0 + wave_n * TN + 4 * (lane >> 4);
    if (g.split == 1) {
        if (g.d_stage) {
            // every wave has passed the last stage's barrier (after waiting
            // for its loads): the operand buffers are free; each wave takes
            // a private TM x TN bf16 region
            constexpr int REG = TM * TN * 2;
            constexpr int RPA = A_STAGE / REG, RPB = B_STAGE / REG;
            static_assert(NW <= 2 * RPA + 2 * RPB, "staging regions fit the operand buffers");
            uint8_t *buf;
            if (wave < RPA)
                buf = s_a0 + wave * REG;
            else if (wave < 2 * RPA)
                buf = s_a1 + (wave - RPA) * REG;
            else if (wave < 2 * RPA + RPB)
                buf = s_b0 + (wave - 2 * RPA) * REG;
            else
                buf = s_b1 + (wave - 2 * RPA - RPB) * REG;
            store_tile_staged<FM, FN>(ep, m0 + wave_m * TM, n0 + wave_n * TN, acc, buf);
            return;
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                store_quad(ep, mb + fm * 16, nb + fn * 16, acc[fn][fm]);
        return;
    }
    if (g.split_atomic) {
        // bf16-atomic reduction (opt-in): D already holds bf16(beta * C)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                atomic_add_quad(ep, mb + fm * 16, nb + fn * 16, acc[fn][fm]);
        return;
    }
    // fp32 partial tile of this K chunk: [tile][z][wave][fn][fm][lane] float4s
    constexpr uint32_t PART = BM * BN * 4;  // bytes per partial tile
    const auto rws = make_rsrc_u(g.ws + (size_t)t * g.split * (BM * BN), (uint32_t)(g.split * PART));
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            store16_coherent(rws, z * PART + (uint32_t)((((wave * FN + fn) * FM + fm) * 64 + lane) * 16),
                             acc[fn][fm]);
    // (the dense FP6 tile's operand buffers fill the LDS: its flag takes a
    // word of the A buffer, free after the last stage's barrier)
    if (!(A6D ? split_arrive_last_via(g.counters + t, g.split, reinterpret_cast<int *>(s_a0))
              : split_arrive_last(g.counters + t, g.split)))
        return;
    // per group of up to four fragments of a column, every fragment's
    // partial of a chunk is requested before any is added (one memory
    // latency per chunk and group, not per fragment); each element adds the
    // chunks in z order
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

// D = bf16(beta * C), or +0 when beta == 0: the starting value the
// bf16-atomic split-K reduction adds its chunks onto.  One thread per pair
// of columns (ldd and N are even there).
__global__ void __launch_bounds__(256) mx_d_init_kernel(GemmArgs g)
{
    const int64_t pairs = (int64_t)g.M * (g.N / 2);
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= pairs)
        return;
    const int m = (int)(i / (g.N / 2)), n = (int)(i - (int64_t)m * (g.N / 2)) * 2;
    float v0 = 0.0f, v1 = 0.0f;
    if (g.beta != 0.0f) {
        if (g.c_f32) {
            const float *c = reinterpret_cast<const float *>(g.C) + (int64_t)m * g.ldc + n;
            v0 = g.beta * c[0];
            v1 = g.beta * c[1];
        } else {
            const uint16_t *c = reinterpret_cast<const uint16_t *>(g.C) + (int64_t)m * g.ldc + n;
            v0 = g.beta * bf16_to_f32(c[0]);
            v1 = g.beta * bf16_to_f32(c[1]);
        }
    }
    *reinterpret_cast<uint32_t *>(g.D + (int64_t)m * g.ldd + n) = bf16x2_rne(v0, v1);
}

void launch_d_init(const GemmArgs &g, hipStream_t s)
{
    const int64_t pairs = (int64_t)g.M * (g.N / 2);
    hipLaunchKernelGGL(mx_d_init_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, s, g);
}

template <int BM, int BN, int WM, int WN, int BLAY, bool SAPACK>
static void launch_tile(const GemmArgs &g, int grid, hipStream_t s)
{
    constexpr bool SBPACK = BLAY == 1 || BLAY == 3;
    // SVEC: whole 8-block stages and 8-byte scale-row loads (packed scales
    // need only the former)
    const bool sa_ok = SAPACK ? g.KB % 8 == 0 : g.sa_fast != 0;
    const bool sb_ok = SBPACK ? g.KB % 8 == 0 : g.sb_fast != 0;
    // persistent form: 256 x 256 with packed A and B scales, B's codes
    // packed or MN-major (its other layouts spill in the tile loop; the
    // 256 x 128 tile and the 8-bit 128 x 256 tile measured no faster
    // persistent)
    if constexpr (BM == 256 && BN == 256 && (BLAY == 1 || BLAY == 3) && SAPACK) {
        if (g.persist_grid > 0 && sa_ok && sb_ok) {
            hipLaunchKernelGGL((mx_tile_kernel<BM, BN, WM, WN, BLAY, true, SAPACK, 0, true>), dim3(g.persist_grid),
                               dim3(64 * WM * WN), 0, s, g);
            return;
        }
    }
    if (sa_ok && sb_ok)
        hipLaunchKernelGGL((mx_tile_kernel<BM, BN, WM, WN, BLAY, true, SAPACK>), dim3(grid), dim3(64 * WM * WN), 0, s, g);
    else
        hipLaunchKernelGGL((mx_tile_kernel<BM, BN, WM, WN, BLAY, false, SAPACK>), dim3(grid), dim3(64 * WM * WN), 0, s, g);
}

// 8-bit A (FP8 E4M3 / BF8 E5M2), row-major A scales
template <int BM, int BN, int WM, int WN, bool BPACK, int AFMT>
static void launch_tile_a8(const GemmArgs &g, int grid, hipStream_t s)
{
    constexpr int BLAY = BPACK ? 1 : 0;
    if (g.sa_fast && (BPACK ? g.KB % 8 == 0 : g.sb_fast != 0))
        hipLaunchKernelGGL((mx_tile_kernel<BM, BN, WM, WN, BLAY, true, false, AFMT>), dim3(grid), dim3(64 * WM * WN), 0, s, g);
    else
        hipLaunchKernelGGL((mx_tile_kernel<BM, BN, WM, WN, BLAY, false, false, AFMT>), dim3(grid), dim3(64 * WM * WN), 0, s, g);
}

// FP6 A in the dense operand order (launch_fp6_pack), packed B and packed A
// scales; SVEC: whole 8-block stages; persistent under the conditions of the
// FP4 256 x 256 tile
template <int BM, int BN, int WM, int WN, int AFMT>
static void launch_tile_fp6_dense(const GemmArgs &g, int grid, hipStream_t s)
{
    if (g.persist_grid > 0 && g.KB % 8 == 0)
        hipLaunchKernelGGL((mx_tile_kernel<BM, BN, WM, WN, 1, true, true, AFMT, true, true>), dim3(g.persist_grid),
                           dim3(64 * WM * WN), 0, s, g);
    else if (g.KB % 8 == 0)
        hipLaunchKernelGGL((mx_tile_kernel<BM, BN, WM, WN, 1, true, true, AFMT, false, true>), dim3(grid),
                           dim3(64 * WM * WN), 0, s, g);
    else
        hipLaunchKernelGGL((mx_tile_kernel<BM, BN, WM, WN, 1, false, true, AFMT, false, true>), dim3(grid),
                           dim3(64 * WM * WN), 0, s, g);
}

#define MX_TILE_A8(BM, BN, WM, WN, OCC)                                                                    \
    {BM, BN, OCC,                                                                                          \
     {launch_tile_a8<BM, BN, WM, WN, false, 1>, launch_tile_a8<BM, BN, WM, WN, false, 2>,                  \
      launch_tile_a8<BM, BN, WM, WN, false, 3>, launch_tile_a8<BM, BN, WM, WN, false, 4>},                 \
     {launch_tile_a8<BM, BN, WM, WN, true, 1>, launch_tile_a8<BM, BN, WM, WN, true, 2>,                    \
      launch_tile_a8<BM, BN, WM, WN, true, 3>, launch_tile_a8<BM, BN, WM, WN, true, 4>}, "tile_a8_" #BM "x" #BN, \
     false}

const TileKernelA8 *tile_kernels_a8(int *count)
{
    // the dense FP6 tile: 8 waves of 64 x 128 (four A fragments of 24 bytes
    // and eight B fragments per step, the registers the FP4 tile's 128 x 64
    // waves use)
    static const TileKernelA8 table[] = {
        MX_TILE_A8(128, 256, 2, 4, 1),
        MX_TILE_A8(128, 128, 2, 2, 1),
        MX_TILE_A8(64, 64, 2, 2, 3),
        {256, 256, 1, {nullptr, nullptr, nullptr, nullptr},
         {nullptr, nullptr, launch_tile_fp6_dense<256, 256, 4, 2, 3>, launch_tile_fp6_dense<256, 256, 4, 2, 4>},
         "tile_fp6_256x256", true},
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}
#undef MX_TILE_A8

#define MX_TILE(BM, BN, WM, WN, OCC, DEEP)                                                              \
    {BM, BN, OCC, launch_tile<BM, BN, WM, WN, 0, false>, launch_tile<BM, BN, WM, WN, 1, false>,         \
     launch_tile<BM, BN, WM, WN, 1, true>, launch_tile_deep<BM, BN, WM, WN, false, false>,              \
     launch_tile_deep<BM, BN, WM, WN, true, false>, launch_tile_deep<BM, BN, WM, WN, true, true>,       \
     launch_tile<BM, BN, WM, WN, 2, false>, launch_tile<BM, BN, WM, WN, 3, false>,                      \
     launch_tile<BM, BN, WM, WN, 3, true>, DEEP, "tile_" #BM "x" #BN}

const TileKernel *tile_kernels(int *count)
{
    static const TileKernel table[] = {
        MX_TILE(256, 256, 2, 4, 1, false),
        MX_TILE(256, 128, 2, 2, 1, false),
        MX_TILE(128, 128, 2, 2, 2, false),
        MX_TILE(64, 64, 2, 2, 4, true),
    };
#undef MX_TILE
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace mx

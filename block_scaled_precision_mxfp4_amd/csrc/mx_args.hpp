// Kernel arguments and launcher table shared by the host library and the
// gfx950 kernels.  Host-side only plain types; no torch, no device code.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace mx {

struct GemmArgs {
    uint16_t *D;          // bf16 [M][ldd]
    const void *C;        // bf16 or f32 (c_f32) [M][ldc], read only when beta != 0
    const uint8_t *A;     // fp4x2 [M][lda_b]
    const uint8_t *B;     // fp4x2 [N][ldb_b], or the packed layout
    const uint8_t *SA;    // E8M0 [M][ldsa], or the packed scale layout
    const uint8_t *SB;    // E8M0 [N][ldsb], or the packed layout
    float *ws;            // split-K fp32 partials
    int *counters;        // split-K arrival counters, one per output tile, zero between calls
    float alpha, beta;
    int M, N, K;
    int KB;               // K / 32 scale blocks
    int64_t lda_b, ldb_b; // byte pitch of A and B rows
    int64_t ldsa, ldsb;   // byte pitch of scale rows
    int64_t ldc, ldd;     // element pitch of C and D rows
    int split;            // K chunks (1 = no split)
    int kb_per_split;     // K-blocks per chunk, a multiple of 8
    int tiles_m, tiles_n; // output tiles per dimension
    int ks_total;         // packed B: 128-K steps per 16-row group, ceil(KB/4)
    int sn8;              // packed scales: (KB rounded up to 8) / 8
    int sa_fast, sb_fast; // scale rows allow aligned 8-byte loads (tiled kernel)
    int scale16;          // both scale operands allow aligned 16-byte row groups (skinny kernel)
    int d_vec, c_vec;     // 8-byte D stores / C loads allowed
    int d_stage;          // beta == 0, D 16-byte aligned, ldd % 8 == 0: LDS-staged epilogue
    int sa_packed;        // scaleA in the packed scale layout
    int sa16, sb16;       // row-major scale rows in 16-byte aligned groups of 16 K-blocks
    int group_m;          // tile-order grouping along M
    int c_f32;            // C holds float32 elements
    int split_atomic;     // split > 1: chunks add bf16(alpha * partial) into D with bf16 atomics
    int persist_grid;     // > 0: the 256x256 tiled kernel runs persistent with this many workgroups
};

typedef void (*LaunchFn)(const GemmArgs &, int grid, hipStream_t);

// Tiled kernel (operands staged through LDS): tile shapes available.
struct TileKernel {
    int bm, bn;
    int occupancy;        // workgroups per CU the kernel's LDS allows
    // two-stage kernel (any strides); four-slot ring (dword-aligned scale
    // rows, K % 128 == 0).  plain: row-major B and scales; packed: packed B
    // and B scales; packed_sa: packed B, B scales and A scales
    LaunchFn plain, packed, packed_sa;
    LaunchFn deep_plain, deep_packed, deep_packed_sa;
    // two-stage kernel with MN-major B codes ([K][N], N contiguous): B
    // scales row-major; B scales packed; B and A scales packed
    LaunchFn kn, kn_packed_sb, kn_packed_sa;
    bool prefer_deep;                  // the ring kernel is the faster one for this tile
    const char *name;
};

template <int BM, int BN, int WM, int WN, bool BPACK, bool SAPACK>
void launch_tile_deep(const GemmArgs &g, int grid, hipStream_t s);
// Host-side table of the tiled kernels, in the planner's preference order.
const TileKernel *tile_kernels(int *count);

// Tiled kernel with 8-bit A (FP8 E4M3, BF8 E5M2, or FP6 E2M3 / E3M2 in the
// padded layout of launch_fp6_pad; B FP4, row-major A scales): launchers
// indexed by a_format - 1
struct TileKernelA8 {
    int bm, bn;
    int occupancy;
    LaunchFn plain[4], packed[4];
    const char *name;
    // FP6 A only, in the dense operand order of launch_fp6_pack (g.lda_b =
    // bytes per 16-row group), with packed B and packed A scales: launchers
    // packed[2], packed[3]; the others are null
    bool fp6_dense;
};
const TileKernelA8 *tile_kernels_a8(int *count);

// Skinny kernel (M <= 64, B streamed from memory into registers).
// index: (mg - 1) * 3 + nr_index with nr in {1, 2, 4}.
struct SkinnyKernel {
    int mg, nr;
    LaunchFn plain, packed, packed_sa;
    const char *name;
};
const SkinnyKernel *skinny_kernels(int *count);
// The skinny kernel with one 16-row group (M <= 16) and NR = 1 for A in a
// wider format (a_fmt 1..4: FP8 E4M3, BF8 E5M2, FP6 E2M3, FP6 E3M2), B FP4.
void launch_skinny_wide(int a_fmt, bool b_packed, const GemmArgs &g, int grid, hipStream_t s);
// M == 1 with a bf16 A row quantized to MXFP4 on load (g.A = the row,
// g.lda_b its byte pitch; g.SA unused); nr = 1, 2 or 4 as planned
void launch_skinny_bf16a(int nr, bool b_packed, const GemmArgs &g, int grid, hipStream_t s);

// Skinny kernel for 16 < M <= 64 with the waves splitting B's rows and A
// staged once per workgroup in LDS: mg 16-row groups of A, nrw 16-row groups
// of B per wave; launchers and names per A format (index a_format: FP4, FP8
// E4M3, BF8 E5M2, FP6 E2M3, FP6 E3M2).  index: mg - 2.
struct RowsKernel {
    int mg, nrw;
    LaunchFn plain[5], packed[5];
    const char *name[5];
    // FP4 A, row-major B, a ring of two slots: two workgroups fit a CU's
    // LDS, for grids with more workgroups than CUs
    LaunchFn lean;
    const char *lean_name;
};
const RowsKernel *rows_kernels(int *count);

void launch_pack_b(uint8_t *Bp, const uint8_t *B, int N, int KB, int64_t ldb_b, hipStream_t s);
// p[0 .. words) = 0, on stream s
void launch_zero_words(uint32_t *p, size_t words, hipStream_t s);

// bf16 -> MXFP4 quantizer: X [M][ldx] bf16 -> A [M][lda_b] bytes, S [M][lds].
struct QuantArgs {
    const uint16_t *X;
    uint8_t *A;
    uint8_t *S;
    int M, K;
    int64_t ldx, lda_b, lds;
    int64_t blocks;  // M * K / 32
};
int64_t quant_grid(int64_t blocks);  // workgroups launch_quant needs
void launch_quant(const QuantArgs &q, int64_t grid, hipStream_t s);
// Scale shuffle of rows x KB scale bytes (either operand's scales).
void launch_pack_sb(uint32_t *SBp, const uint8_t *SB, int N, int KB, int64_t ldsb, hipStream_t s);
// FP16 GEMM (transposed LDS reads of a K-major B): C = A x B, fp32 out
struct F16Args {
    const uint8_t *A;  // fp16 [M][lda_b bytes]
    const uint8_t *B;  // fp16 [K][ldb_b bytes]
    float *C;          // fp32 [M][ldc]
    int M, N, K;
    int64_t lda_b, ldb_b, ldc;
    int tiles_m, tiles_n;
};
int64_t f16_grid(int M, int N);
void launch_f16(const F16Args &a, int64_t grid, hipStream_t s);

// bf16-atomic split-K: D = bf16(beta * C) (0 when beta == 0) before the
// chunks add into it
void launch_d_init(const GemmArgs &g, hipStream_t s);

// Streaming read of `bytes` (a multiple of 16, below 2^31) from src; sink
// receives at most one word
int64_t stream_read_grid(size_t bytes);
void launch_stream_read(const uint8_t *src, size_t bytes, uint32_t *sink, hipStream_t s);

// Fixed device scratch of the allocation-free entry point (mx_scratch.hip):
// kScratchBytes per device; the first kScratchCounterBytes hold split-K
// arrival counters, the rest partial sums and FP6 A's re-laid copy.
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr size_t kScratchCounterBytes = (size_t)64 << 10;
// This device's scratch address (looked up once per device, with the device
// current); never the array's host-side name.
hipError_t scratch_address(void **ptr);

// FP6 A (rows of lda_b bytes, lda_b % 8 == 0) -> the padded layout the
// 8-bit tiled kernel reads with A's FP6 format code (32 bytes per K-block,
// rows of fp6_pad_pitch(K) bytes) in `out`; codes unchanged
int64_t fp6_pad_pitch(int K);
void launch_fp6_pad(const uint8_t *A, int64_t lda_b, uint8_t *out, int M, int K, hipStream_t s);
// FP6 A -> the dense operand order of the 256 x 256 FP6 tile: per 16-row
// group, fp6_pack_steps(K) 128-K steps of 1536 bytes (the 64 lanes' 24-byte
// operands), fp6_pack_group_bytes(K) per group; zeros past M and K.  The A
// scales (rows of ldsa bytes) go to sa_out in the shuffled scale layout.
int fp6_pack_steps(int K);
int64_t fp6_pack_group_bytes(int K);
void launch_fp6_pack(const uint8_t *A, int64_t lda_b, const uint8_t *SA, int64_t ldsa, uint8_t *out,
                     uint32_t *sa_out, int M, int K, hipStream_t s);

}  // namespace mx

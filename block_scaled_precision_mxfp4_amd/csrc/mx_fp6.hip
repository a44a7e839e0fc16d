// FP6 A (E2M3 or E3M2) re-laid for the tiled kernels, codes unchanged: the
// padded layout of the 8-bit tiles, and the dense operand order of the
// 256 x 256 FP6 tile (below).
//
// The scaled matrix instruction takes FP6 operands at the FP4 rate ("CDNA4
// dense MFMA builtins", "Instruction throughput"): a lane's operand is the 32
// codes of one K-block, 24 bytes of the little-endian 6-bit stream.  A 24-byte
// block does not tile into the 16-byte direct-to-LDS loads, so each block is
// copied into a 32-byte slot laid out exactly like an FP8 operand: per 128-K
// step (4 blocks, 128 bytes) block g's bytes 0..15 go to bytes 16g..16g+15
// and its bytes 16..23 (then 8 zero bytes) to bytes 64+16g..64+16g+15.  The
// 8-bit tiled kernel reads those two 16-byte pieces for lane group g (the
// places an FP8 operand's two 16-element runs occupy) and hands the first
// 24 bytes to the instruction with A's FP6 format code.  Rows are rounded up
// to whole 128-byte steps; one thread per block.
#include "libmxgemm.h"
#include "mx_args.hpp"
#include "mx_device.hpp"

namespace mx {

__global__ void __launch_bounds__(256) mx_fp6_pad_kernel(const uint8_t *__restrict__ A, int64_t lda_b,
                                                         uint8_t *__restrict__ out, int64_t ld_out, int M, int KB)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * KB)
        return;
    const int r = (int)(i / KB), b = (int)(i - (int64_t)r * KB);
    // 24 bytes at an 8-byte aligned offset (the host requires lda_b % 8 == 0)
    const v2u *src = reinterpret_cast<const v2u *>(A + (int64_t)r * lda_b + (int64_t)b * 24);
    const v2u w0 = src[0], w1 = src[1], w2 = src[2];
    uint8_t *dst = out + (int64_t)r * ld_out + (int64_t)(b >> 2) * 128 + (b & 3) * 16;
    *reinterpret_cast<v4i *>(dst) = v4i{(int)w0[0], (int)w0[1], (int)w1[0], (int)w1[1]};
    *reinterpret_cast<v4i *>(dst + 64) = v4i{(int)w2[0], (int)w2[1], 0, 0};
}

int64_t fp6_pad_pitch(int K) { return (int64_t)(K + 127) / 128 * 128; }

void launch_fp6_pad(const uint8_t *A, int64_t lda_b, uint8_t *out, int M, int K, hipStream_t s)
{
    const int KB = K / 32;
    const int64_t threads = (int64_t)M * KB;
    hipLaunchKernelGGL(mx_fp6_pad_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, A, lda_b, out,
                       fp6_pad_pitch(K), M, KB);
}

// Dense operand order for the 256 x 256 tile: per 16-row group and 128-K
// step, the 64 lanes' 24-byte operands back to back (lane l: row l % 16 of
// the group, K-block l / 16 of the step), 1536 bytes; the steps of a group
// follow each other, so a 256-K stage of a group is 3 KiB in one run and
// every direct-to-LDS load a whole 1 KiB.  Steps are counted up to an even
// number; rows past M and K-blocks past K are zero.
//
// A workgroup moves 32 rows x 4 steps: the rows' 384-byte runs are read in
// 16-byte pieces (24 consecutive threads per row, streaming loads; 8-byte
// pieces when the row pitch is not a multiple of 16) whose 8-byte words are
// dropped into LDS at their operand-order places, then each of the two
// groups' 6 KiB runs is written with 16-byte stores.  The same workgroup writes the A scales of
// its 32 rows and two 8-block steps in the shuffled scale layout (the one
// mxgemm_pack_scales writes: word (row group, step, lane) holds rows 16j +
// lane % 16 at K-block 4i + lane / 16 of the step, byte 2i + j; 0x7F past M
// and K).
template <bool V16>
__global__ void __launch_bounds__(256) mx_fp6_pack_kernel(const uint8_t *__restrict__ A, int64_t lda_b,
                                                          const uint8_t *__restrict__ SA, int64_t ldsa,
                                                          uint8_t *__restrict__ out, uint32_t *__restrict__ sa_out,
                                                          int M, int KB, int ks_pad)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_out[2 * 4 * 1536];
    const int quads = (ks_pad + 3) / 4;
    const int g32 = blockIdx.x / quads, s0 = (blockIdx.x - g32 * quads) * 4;
    const int tid = threadIdx.x;
    // the A-scale bytes of this thread's shuffled word (threads 0-127: two
    // 8-block steps x 64 lanes), loaded before the operand bytes so that
    // their latency overlaps the operands' instead of following it
    const int d3 = s0 / 2 + (tid >> 6), slane = tid & 63;
    const bool sc_on = tid < 128 && d3 < ks_pad / 2;
    uint32_t sb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = g32 * 32 + (j & 1) * 16 + (slane & 15);
        const int col = d3 * 8 + (j >> 1) * 4 + (slane >> 4);
        sb[j] = sc_on && row < M && col < KB ? SA[(int64_t)row * ldsa + col] : 0x7Fu;
    }
    // word w (of 12) of step s of row r -> its place in the group's run
    auto place = [&](int r, int s, int w, v2u v) __attribute__((always_inline)) {
        const int l = (w / 3) * 16 + (r & 15);
        *reinterpret_cast<v2u *>(s_out + (r >> 4) * 6144 + s * 1536 + l * 24 + (w % 3) * 8) = v;
    };
    if constexpr (V16) {
#pragma unroll
        for (int pass = 0; pass < 3; ++pass) {
            const int q = pass * 256 + tid;  // 32 rows x 24 pieces
            const int r = q / 24, c = q - r * 24;
            const int s = c / 6, w = (c % 6) * 2;  // step of the four, first word of the piece in it
            const int row = g32 * 32 + r, blk0 = 4 * (s0 + s) + w / 3, blk1 = 4 * (s0 + s) + (w + 1) / 3;
            const uint8_t *src = A + (int64_t)row * lda_b + (int64_t)(s0 + s) * 96 + w * 8;
            v2u lo = v2u{0u, 0u}, hi = v2u{0u, 0u};
            if (row < M && blk1 < KB) {
                const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(src));
                lo = v2u{(uint32_t)v[0], (uint32_t)v[1]};
                hi = v2u{(uint32_t)v[2], (uint32_t)v[3]};
            } else if (row < M && blk0 < KB) {
                lo = *reinterpret_cast<const v2u *>(src);
            }
            place(r, s, w, lo);
            place(r, s, w + 1, hi);
        }
    } else {
#pragma unroll
        for (int pass = 0; pass < 6; ++pass) {
            const int q = pass * 256 + tid;  // 32 rows x 48 words
            const int r = q / 48, wr = q - r * 48;
            const int s = wr / 12, w = wr % 12;  // step of the four, word of the row's 96 bytes in it
            const int row = g32 * 32 + r, blk = 4 * (s0 + s) + w / 3;
            v2u v = v2u{0u, 0u};
            if (row < M && blk < KB)
                v = *reinterpret_cast<const v2u *>(A + (int64_t)row * lda_b + (int64_t)(s0 + s) * 96 + w * 8);
            place(r, s, w, v);
        }
    }
    if (sc_on)
        sa_out[((int64_t)g32 * (ks_pad / 2) + d3) * 64 + slane] = sb[0] | sb[1] << 8 | sb[2] << 16 | sb[3] << 24;
    __syncthreads();
    const int groups = (M + 15) / 16;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int q = pass * 256 + tid;  // 768 chunks of 16 bytes
        const int gi = q / 384, off = (q - gi * 384) * 16;
        const int grp = g32 * 2 + gi, s = s0 + off / 1536;
        if (grp < groups && s < ks_pad)
            *reinterpret_cast<v4i *>(out + ((int64_t)grp * ks_pad + s0) * 1536 + off) =
                *reinterpret_cast<const v4i *>(s_out + gi * 6144 + off);
    }
}

int fp6_pack_steps(int K) { return (K / 32 + 7) / 8 * 2; }
int64_t fp6_pack_group_bytes(int K) { return (int64_t)fp6_pack_steps(K) * 1536; }

void launch_fp6_pack(const uint8_t *A, int64_t lda_b, const uint8_t *SA, int64_t ldsa, uint8_t *out,
                     uint32_t *sa_out, int M, int K, hipStream_t s)
{
    const int ks_pad = fp6_pack_steps(K);
    const int64_t grid = (int64_t)((M + 31) / 32) * ((ks_pad + 3) / 4);
    // (A is 16-byte aligned; 16-byte pieces need 16-byte rows as well)
    if (lda_b % 16 == 0)
        hipLaunchKernelGGL(mx_fp6_pack_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, A, lda_b, SA, ldsa, out,
                           sa_out, M, K / 32, ks_pad);
    else
        hipLaunchKernelGGL(mx_fp6_pack_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, A, lda_b, SA, ldsa, out,
                           sa_out, M, K / 32, ks_pad);
}

}  // namespace mx

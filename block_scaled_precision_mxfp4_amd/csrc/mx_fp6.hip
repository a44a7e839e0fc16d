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

// Dense operand order for the 256 x 256 tile: per 16-row group and 128-K
// step, the 64 lanes' 24-byte operands back to back (lane l: row l % 16 of
// the group, K-block l / 16 of the step), 1536 bytes; the steps of a group
// follow each other, so a 256-K stage of a group is 3 KiB in one run and
// every direct-to-LDS load a whole 1 KiB.  Steps are counted up to an even
// number; rows past M and K-blocks past K are zero.  A workgroup copies four
// steps of one group, 8 bytes per thread and pass: 48 consecutive threads
// read one row's 384 contiguous bytes.
__global__ void __launch_bounds__(256) mx_fp6_pack_kernel(const uint8_t *__restrict__ A, int64_t lda_b,
                                                          uint8_t *__restrict__ out, int M, int KB, int ks_pad)
{
    const int quads = (ks_pad + 3) / 4;
    const int grp = blockIdx.x / quads, s0 = (blockIdx.x - grp * quads) * 4;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int q = pass * 256 + threadIdx.x;  // 16 rows x 48 words
        const int r = q / 48, wr = q - r * 48;
        const int s = s0 + wr / 12, w = wr % 12;  // step, word of the row's 96 bytes in it
        if (s >= ks_pad)
            continue;
        const int row = grp * 16 + r, blk = 4 * s + w / 3;
        v2u v = v2u{0u, 0u};
        if (row < M && blk < KB)
            v = *reinterpret_cast<const v2u *>(A + (int64_t)row * lda_b + (int64_t)s * 96 + w * 8);
        const int l = (w / 3) * 16 + r;
        *reinterpret_cast<v2u *>(out + ((int64_t)grp * ks_pad + s) * 1536 + l * 24 + (w % 3) * 8) = v;
    }
}

int fp6_pack_steps(int K) { return (K / 32 + 7) / 8 * 2; }
int64_t fp6_pack_group_bytes(int K) { return (int64_t)fp6_pack_steps(K) * 1536; }

void launch_fp6_pack(const uint8_t *A, int64_t lda_b, uint8_t *out, int M, int K, hipStream_t s)
{
    const int ks_pad = fp6_pack_steps(K);
    const int64_t grid = (int64_t)((M + 15) / 16) * ((ks_pad + 3) / 4);
    hipLaunchKernelGGL(mx_fp6_pack_kernel, dim3((unsigned)grid), dim3(256), 0, s, A, lda_b, out, M, K / 32, ks_pad);
}

void launch_fp6_pad(const uint8_t *A, int64_t lda_b, uint8_t *out, int M, int K, hipStream_t s)
{
    const int KB = K / 32;
    const int64_t threads = (int64_t)M * KB;
    hipLaunchKernelGGL(mx_fp6_pad_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, A, lda_b, out,
                       fp6_pad_pitch(K), M, KB);
}

}  // namespace mx

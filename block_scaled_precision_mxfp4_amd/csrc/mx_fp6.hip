// FP6 A -> FP8 A, exactly, for the 8-bit tiled kernel.
//
// Every FP6 value is an FP8 value of the matching shape: E2M3 (bias 1,
// subnormals m * 2^-3, largest 7.5) lies inside E4M3 (bias 7, normals down
// to 2^-6), and E3M2 (bias 3, subnormals m * 2^-4, largest 28) inside E5M2
// (bias 15).  The element encodings are those of the OCP Microscaling
// Formats v1.0 specification; the pages list FP6 E2M3 / E3M2 and FP8 E4M3 /
// E5M2 as inputs of the same scaled matrix instruction ("CDNA4 dense MFMA
// builtins", "Mixed-precision with scaling").  With the E8M0 scales left as
// they are, the instruction then multiplies the same values.
//
// One thread per 16 elements of a row: 12 bytes of the little-endian 6-bit
// stream in (three dword loads), 16 FP8 bytes out (one 16-byte store).
#include "libmxgemm.h"
#include "mx_args.hpp"
#include "mx_device.hpp"

namespace mx {

// E2M3 code -> E4M3 code
__device__ __forceinline__ uint32_t e2m3_to_e4m3(uint32_t c)
{
    const uint32_t s = (c >> 5) << 7, e = (c >> 3) & 3, m = c & 7;
    if (e != 0)
        return s | ((e + 6) << 3) | m;  // (1 + m/8) 2^(e-1): exponent field e - 1 + 7
    if (m == 0)
        return s;
    // m 2^-3 = (1 + f) 2^p with p = floor(log2 m): exponent field p - 3 + 7
    const uint32_t p = 31 - __builtin_clz(m);
    return s | ((p + 4) << 3) | ((m << (3 - p)) & 7);
}

// E3M2 code -> E5M2 code
__device__ __forceinline__ uint32_t e3m2_to_e5m2(uint32_t c)
{
    const uint32_t s = (c >> 5) << 7, e = (c >> 2) & 7, m = c & 3;
    if (e != 0)
        return s | ((e + 12) << 2) | m;  // (1 + m/4) 2^(e-3): exponent field e - 3 + 15
    if (m == 0)
        return s;
    // m 2^-4 = (1 + f) 2^p with p = floor(log2 m): exponent field p - 4 + 15
    const uint32_t p = 31 - __builtin_clz(m);
    return s | ((p + 11) << 2) | ((m << (2 - p)) & 3);
}

template <int FMT>
__global__ void __launch_bounds__(256) mx_fp6_to_fp8_kernel(const uint8_t *__restrict__ A, int64_t lda_b,
                                                            uint8_t *__restrict__ out, int M, int K)
{
    const int per_row = K / 16;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * per_row)
        return;
    const int r = (int)(i / per_row), q = (int)(i - (int64_t)r * per_row);
    const uint32_t *src = reinterpret_cast<const uint32_t *>(A + (int64_t)r * lda_b + (int64_t)q * 12);
    const uint64_t lo = (uint64_t)src[0] | ((uint64_t)src[1] << 32);
    const uint32_t hi = src[2];
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        // bits 6j .. 6j+5 of the 96-bit stream lo | hi << 64
        uint32_t c;
        if (6 * j + 6 <= 64)
            c = (uint32_t)(lo >> (6 * j)) & 63u;
        else if (6 * j >= 64)
            c = (hi >> (6 * j - 64)) & 63u;
        else
            c = ((uint32_t)(lo >> (6 * j)) | (hi << (64 - 6 * j))) & 63u;
        const uint32_t o = FMT == MXGEMM_FMT_FP6_E2M3 ? e2m3_to_e4m3(c) : e3m2_to_e5m2(c);
        w[j >> 2] |= o << (8 * (j & 3));
    }
    *reinterpret_cast<v4i *>(out + (int64_t)r * K + (int64_t)q * 16) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
}

void launch_fp6_to_fp8(int a_fmt, const uint8_t *A, int64_t lda_b, uint8_t *out, int M, int K, hipStream_t s)
{
    const int64_t threads = (int64_t)M * (K / 16);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (a_fmt == MXGEMM_FMT_FP6_E2M3)
        hipLaunchKernelGGL(mx_fp6_to_fp8_kernel<MXGEMM_FMT_FP6_E2M3>, grid, dim3(256), 0, s, A, lda_b, out, M, K);
    else
        hipLaunchKernelGGL(mx_fp6_to_fp8_kernel<MXGEMM_FMT_FP6_E3M2>, grid, dim3(256), 0, s, A, lda_b, out, M, K);
}

}  // namespace mx

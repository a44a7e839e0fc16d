// bf16 -> MXFP4 activation quantizer on gfx950.
//
// Produces the operand format the GEMM reads ("Data layouts" of the
// asm_f4gemm README: packed E2M1 codes, low nibble = even k, one E8M0 scale
// per 32 consecutive K elements of a row).  The pages do not say how a
// scale is chosen for real-valued input; this follows the conversion rule
// of the OCP Microscaling Formats v1.0 specification (section 6.3):
//   - scale exponent X = floor(log2 max|v|) - 2, clamped to [-127, 127]
//     (2 is the largest E2M1 exponent: 6 = 1.5 * 2^2);
//   - each element v / 2^X rounded to the nearest E2M1 value, ties to the
//     even mantissa, saturating at 6, sign kept (a negative value that
//     rounds to zero is code 0x8);
//   - a block holding a NaN or an infinity gets scale 0xFF and codes 0;
//     an all-zero block gets scale 0x00 and codes 0.
//
// Bound by HBM: 2 bytes read and 17/32 byte written per element.  Four
// lanes share a block, each holding 8 consecutive elements (one 16-byte
// load); the block maximum and the NaN/inf flag are combined across the
// four lanes with two cross-lane exchanges; each lane writes its 8 codes as
// one 32-bit word and the first lane of the four writes the scale byte.
// Input and codes pass through once, so both go with the non-temporal hint
// (the caches need not keep them).
#include "mx_args.hpp"
#include "mx_device.hpp"
#include "mx_quantize.hpp"

namespace mx {

// A workgroup takes 64*U consecutive blocks: in round u, the four lanes
// 4g..4g+3 take block base + 64u + g, so each load instruction of a wave
// covers 16 consecutive blocks (1 KiB of a row).  All U loads are issued
// before the first block is encoded.
template <int U>
__global__ void __launch_bounds__(256) mx_quant_kernel(QuantArgs q)
{
    const int j = threadIdx.x & 3;
    const int g = threadIdx.x >> 2;
    const int64_t base = (int64_t)blockIdx.x * (64 * U);
    const int kbn = q.K >> 5;
    // (row, block) of round 0 by one division; each later round is 64
    // blocks further: 64 / kbn rows and 64 % kbn blocks, plus a carry
    const int64_t b0 = base + g;
    int64_t row = b0 / kbn;
    int col = (int)(b0 - row * kbn);
    const int drow = 64 / kbn, dcol = 64 % kbn;
    v4i x[U];
    int64_t r[U];
    int kb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool live = base + u * 64 + g < q.blocks;
        r[u] = live ? row : -1;
        kb[u] = col;
        x[u] = live ? __builtin_nontemporal_load(reinterpret_cast<const v4i *>(q.X + row * q.ldx + col * 32 + j * 8)) : v4i{0, 0, 0, 0};
        row += drow;
        col += dcol;
        if (col >= kbn) {
            col -= kbn;
            ++row;
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        uint32_t word;
        uint8_t scale;
        quantize_quarter(x[u], word, scale);
        if (r[u] >= 0) {
            __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(q.A + r[u] * q.lda_b + kb[u] * 16 + j * 4));
            if (j == 0)
                q.S[r[u] * q.lds + kb[u]] = scale;
        }
    }
}

// Blocks per lane group.  With the non-temporal hint on the bf16 loads and
// the code stores (each byte is touched once), four measured faster than
// eight (8192 x 8192 on MI355X, alternating: 29.8-32.3 against
// 31.4-33.7 us; plain loads and stores with eight: 35.0-37.6 us, with
// sixteen 40.4-42.8 us).
constexpr int kQuantU = 4;

int64_t quant_grid(int64_t blocks) { return (blocks + 64 * kQuantU - 1) / (64 * kQuantU); }

void launch_quant(const QuantArgs &q, int64_t grid, hipStream_t s)
{
    hipLaunchKernelGGL(mx_quant_kernel<kQuantU>, dim3((unsigned)grid), dim3(256), 0, s, q);
}

}  // namespace mx

// Skinny MXFP4 GEMM for M <= 64 (decode / GEMV shapes) on gfx950.
//
// Here the whole cost is reading B once from HBM, so the kernel streams B
// straight from memory into registers (16 bytes per lane, one instruction
// operand per 16 rows x 128 K) with several loads in flight per lane, and
// keeps the tiny A in the L2.  Each wave owns 16*NR rows of B (= columns of
// D); its accumulators cover all M <= 16*MG rows of D.  The scaled FP4
// instruction still does the arithmetic: rows of A past M are zero lanes
// (out-of-range loads return zero), which costs nothing here because the
// matrix unit is far from busy when bytes arrive at HBM speed.
//
// Split K spreads one row block over several workgroups; the partial sums
// are combined in fp32 in a fixed order by the last workgroup to arrive (see
// split_arrive_last), in the same launch.
#include "mx_args.hpp"
#include "mx_device.hpp"

namespace mx {

template <int MG, int NR, bool BPACK>
__global__ void __launch_bounds__(256) mx_skinny_kernel(GemmArgs g)
{
    constexpr int RW = 16 * NR;  // B rows per wave
    constexpr int RWG = 4 * RW;  // B rows per workgroup
    constexpr int U = 4;         // 128-K steps loaded per batch
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    const int lg = xcd_remap(blockIdx.x, gridDim.x);
    const int z = lg / g.tiles_n;
    const int t = lg - z * g.tiles_n;
    const int nw = t * RWG + wave * RW;  // first row of B (column of D) of this wave

    const int kb_begin = z * g.kb_per_split;
    const int kb_end = min(g.KB, kb_begin + g.kb_per_split);
    const int ks_begin = kb_begin >> 2, ks_end = (kb_end + 3) >> 2;

    const auto ra = make_rsrc(g.A, (uint32_t)(g.M * g.lda_b));
    const auto rsa = make_rsrc(g.SA, (uint32_t)(g.M * g.ldsa));
    __amdgpu_buffer_rsrc_t rb, rsb;
    int half0 = 0;  // packed scales: which 16-row half of its 32-row group row nw is
    if constexpr (BPACK) {
        const int n16 = nw / 16, g16 = max(0, min(NR, (g.N + 15) / 16 - n16));
        rb = make_rsrc(g.B + (int64_t)n16 * g.ks_total * 1024, (uint32_t)(g16 * g.ks_total * 1024));
        const int n32 = nw / 32;
        const int g32 = max(0, min((nw + RW + 31) / 32 - n32, (g.N + 31) / 32 - n32));
        rsb = make_rsrc(g.SB + (int64_t)n32 * g.sn8 * 256, (uint32_t)(g32 * g.sn8 * 256));
        half0 = n16 & 1;
    } else {
        const int rows = max(0, min(RW, g.N - nw));
        rb = make_rsrc(g.B + (int64_t)nw * g.ldb_b, (uint32_t)(rows * g.ldb_b));
        rsb = make_rsrc(g.SB + (int64_t)nw * g.ldsb, (uint32_t)(rows * g.ldsb));
    }

    v4f acc[NR][MG];
#pragma unroll
    for (int nr = 0; nr < NR; ++nr)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
            acc[nr][mg] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int ks0 = ks_begin; ks0 < ks_end; ks0 += U) {
        v4i bfr[U][NR], afr[U][MG];
        uint32_t sbv[U][NR], sav[U][MG];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ks = ks0 + u;
            const int kb = ks * 4 + (lane >> 4);
            const bool ok = ks < ks_end && kb < kb_end;
#pragma unroll
            for (int nr = 0; nr < NR; ++nr) {
                if constexpr (BPACK) {
                    bfr[u][nr] = load16(rb, ok ? (uint32_t)(((nr * g.ks_total + ks) * 64 + lane) * 16) : kOOB);
                    const int grp = (half0 + nr) >> 1, half = (half0 + nr) & 1;
                    const uint32_t w =
                        load4(rsb, ok ? (uint32_t)(((grp * g.sn8 + (ks >> 1)) * 64 + lane) * 4) : kOOB);
                    sbv[u][nr] = w >> (8 * ((ks & 1) * 2 + half));
                } else {
                    const int row = nr * 16 + (lane & 15);
                    bfr[u][nr] = load16(rb, ok ? (uint32_t)(row * g.ldb_b + kb * 16) : kOOB);
                    sbv[u][nr] = load1(rsb, ok ? (uint32_t)(row * g.ldsb + kb) : kOOB);
                }
            }
#pragma unroll
            for (int mg = 0; mg < MG; ++mg) {
                const int row = mg * 16 + (lane & 15);
                afr[u][mg] = load16(ra, ok ? (uint32_t)(row * g.lda_b + kb * 16) : kOOB);
                sav[u][mg] = load1(rsa, ok ? (uint32_t)(row * g.ldsa + kb) : kOOB);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int nr = 0; nr < NR; ++nr)
#pragma unroll
                for (int mg = 0; mg < MG; ++mg)
                    acc[nr][mg] = mfma_fp4<0, 0>(bfr[u][nr], afr[u][mg], acc[nr][mg], (int)sbv[u][nr],
                                                 (int)sav[u][mg]);
    }

    Epilogue ep{g.D, g.C, g.alpha, g.beta, g.M, g.N, g.ldd, g.ldc, g.d_vec, g.c_vec};
    const int mb = lane & 15;
    const int nb = nw + 4 * (lane >> 4);
    if (g.split == 1) {
#pragma unroll
        for (int nr = 0; nr < NR; ++nr)
#pragma unroll
            for (int mg = 0; mg < MG; ++mg)
                store_quad(ep, mb + mg * 16, nb + nr * 16, acc[nr][mg]);
        return;
    }
    constexpr int PART = RWG * MG * 16;  // floats per workgroup partial
    v4f *part = reinterpret_cast<v4f *>(g.ws + ((size_t)t * g.split + z) * (size_t)PART);
#pragma unroll
    for (int nr = 0; nr < NR; ++nr)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
            part[((wave * NR + nr) * MG + mg) * 64 + lane] = acc[nr][mg];
    if (!split_arrive_last(g.counters + t, g.split))
        return;
    const v4f *base = reinterpret_cast<const v4f *>(g.ws + (size_t)t * g.split * (size_t)PART);
#pragma unroll
    for (int nr = 0; nr < NR; ++nr)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
            const int idx = ((wave * NR + nr) * MG + mg) * 64 + lane;
            v4f s = base[idx];
            for (int zz = 1; zz < g.split; ++zz)
                s += base[(size_t)zz * (PART / 4) + idx];
            store_quad(ep, mb + mg * 16, nb + nr * 16, s);
        }
}

template <int MG, int NR, bool BPACK>
static void launch_skinny(const GemmArgs &g, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((mx_skinny_kernel<MG, NR, BPACK>), dim3(grid), dim3(256), 0, s, g);
}

#define MX_SKINNY(MG, NR) \
    {MG, NR, launch_skinny<MG, NR, false>, launch_skinny<MG, NR, true>, "skinny_m" #MG "x16_n" #NR "x64"}
const SkinnyKernel *skinny_kernels(int *count)
{
    static const SkinnyKernel table[] = {
        MX_SKINNY(1, 1), MX_SKINNY(1, 2), MX_SKINNY(1, 4),
        MX_SKINNY(2, 1), MX_SKINNY(2, 2), MX_SKINNY(2, 4),
        MX_SKINNY(3, 1), MX_SKINNY(3, 2), MX_SKINNY(3, 4),
        MX_SKINNY(4, 1), MX_SKINNY(4, 2), MX_SKINNY(4, 4),
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

void launch_pack_sb(uint32_t *SBp, const uint8_t *SB, int N, int KB, int64_t ldsb, hipStream_t s)
{
    const int sn8 = (KB + 7) / 8;
    const int64_t total = (int64_t)((N + 31) / 32) * sn8 * 64;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(mx_pack_sb_kernel, dim3((unsigned)blocks), dim3(256), 0, s, SBp, SB, N, KB, ldsb, sn8,
                       total);
}

}  // namespace mx

// Streaming-read reference kernel: reads a buffer once with the same 16-byte
// non-temporal buffer loads the skinny kernels stream B with, folding every
// word into a register that decides a store which never happens in practice
// (so no load can be dropped).  Timed beside the M = 1 GEMM it gives the HBM
// read rate this chip reaches for that byte count -- the practical ceiling of
// a kernel whose minimum DRAM traffic ("Optimizing GEMM in HIP", background:
// the GEMM's arithmetic intensity and its minimum required traffic) is that
// many bytes.
#include "mx_args.hpp"
#include "mx_device.hpp"

namespace mx {

constexpr int kStreamThreads = 256;
constexpr int kStreamInFlight = 4;  // 16-byte loads per lane before their use

__global__ void __launch_bounds__(kStreamThreads) mx_stream_read_kernel(const uint8_t *src, uint32_t bytes,
                                                                        uint32_t *sink)
{
    const auto r = make_rsrc(src, bytes);
    const uint32_t stride = gridDim.x * kStreamThreads * 16u;
    uint32_t off = (blockIdx.x * kStreamThreads + threadIdx.x) * 16u;
    v4i acc = {0, 0, 0, 0};
    for (; off < bytes; off += kStreamInFlight * stride) {
        v4i v[kStreamInFlight];
#pragma unroll
        for (int i = 0; i < kStreamInFlight; ++i) {
            const uint32_t o = off + i * stride;  // past the end: zeros, no traffic
            v[i] = load16_stream(r, o < bytes ? o : kOOB);
        }
#pragma unroll
        for (int i = 0; i < kStreamInFlight; ++i)
            acc ^= v[i];
    }
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x5EEDF00D)
        sink[0] = (uint32_t)acc[0];
}

int64_t stream_read_grid(size_t bytes)
{
    // enough workgroups that every lane has its first kStreamInFlight loads
    // in flight at once, up to 8 per compute unit
    const int64_t chunks = (int64_t)(bytes / 16);
    int64_t g = (chunks + kStreamThreads * kStreamInFlight - 1) / (kStreamThreads * kStreamInFlight);
    return g < 1 ? 1 : (g > 2048 ? 2048 : g);
}

void launch_stream_read(const uint8_t *src, size_t bytes, uint32_t *sink, hipStream_t s)
{
    hipLaunchKernelGGL(mx_stream_read_kernel, dim3((unsigned)stream_read_grid(bytes)), dim3(kStreamThreads), 0, s,
                       src, (uint32_t)bytes, sink);
}

}  // namespace mx

// Pipeline helpers for the tiled kernels (gfx950): explicit memory-counter
// waits, stage barriers, and LDS fragment reads issued from inline assembly
// with immediate offsets.
#pragma once

#include "mx_device.hpp"

#include <type_traits>
#include <utility>

namespace mx {

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14;
    // expcnt (bits 6:4) and lgkmcnt (bits 11:8) left at their maxima
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Stage hand-over: this wave's loads of the stage have landed (at most N
// later loads still in flight), its LDS reads of the previous stage are done,
// then the workgroup barrier.  Written as one asm block with a memory clobber
// so that the compiler neither moves memory operations across it nor adds the
// full vmcnt(0) a fenced barrier would imply.
template <int N>
__device__ __forceinline__ void stage_sync()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// LDS reads issued from asm: the compiler's bookkeeping of in-flight
// direct-to-LDS loads only tracks a few of them precisely and would make
// these reads wait for loads into other ring slots.  Their results are used
// only after lds_wait_n(), which waits for them and passes every value
// through as an operand, so no use can be scheduled before the wait.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

template <int OFF>
__device__ __forceinline__ v4i lds_read16(uint32_t base)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    v4i r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(base), "n"(OFF) : "memory");
    return r;
}

template <int OFF>
__device__ __forceinline__ v2u lds_read8(uint32_t base)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    v2u r;
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(base), "n"(OFF) : "memory");
    return r;
}

template <int OFF>
__device__ __forceinline__ uint32_t lds_read4(uint32_t base)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    uint32_t r;
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(base), "n"(OFF) : "memory");
    return r;
}

template <int OFF>
__device__ __forceinline__ uint32_t lds_read1(uint32_t base)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    uint32_t r;
    asm volatile("ds_read_u8 %0, %1 offset:%2" : "=v"(r) : "v"(base), "n"(OFF) : "memory");
    return r;
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ void asm_pass(v4i &r) { asm volatile("" : "+v"(r)); }
__device__ __forceinline__ void asm_pass(v2u &r) { asm volatile("" : "+v"(r)); }
__device__ __forceinline__ void asm_pass(uint32_t &r) { asm volatile("" : "+v"(r)); }
template <typename T, int N>
__device__ __forceinline__ void asm_pass(T (&r)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        asm_pass(r[i]);
}

// Wait until at most N LDS reads are still outstanding, then pass the given
// registers through: reads complete in issue order, so the registers filled by
// all but the last N reads are valid afterwards.
template <int N, typename... T>
__device__ __forceinline__ void lds_wait_n(T &...regs)
{
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
    (asm_pass(regs), ...);
}

__device__ __forceinline__ void load4_to_lds(__amdgpu_buffer_rsrc_t r, lds_void *lds, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, off, 0, 0, 0);
}

}  // namespace mx

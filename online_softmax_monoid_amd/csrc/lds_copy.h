// lds_copy.h -- global -> LDS copies by buffer DMA, issued as inline assembly.
//
// The kernels that include this keep every wait on these copies explicit
// (s_waitcnt vmcnt with a count of the copies that may still be in flight).
// Issued through the compiler builtin instead, the compiler drains in-flight
// copies before each LDS read it cannot prove disjoint from them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor with 32-bit offsets, range-checked against `bytes`:
// bytes at or past it read as zero.
__device__ __forceinline__ u32x4 make_desc(const void *base, uint32_t bytes)
{
    const uint64_t addr = (uint64_t)(uintptr_t)base;
    u32x4 d;
    d.x = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    d.y = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32) & 0xffffu);
    d.z = __builtin_amdgcn_readfirstlane(bytes);
    d.w = 0x00020000u;
    return d;
}

// 16 bytes per lane from global memory (byte offset voffset in the buffer)
// straight into LDS at lds_base + 16 * lane. M0 holds the LDS address. The
// compiler's hazard check does not look inside the assembly, so it carries
// its own wait states: five, the most any of its inputs needs (a descriptor
// word written by a VALU instruction such as v_readfirstlane and read by a
// vector memory instruction; M0 written and read by an LDS copy needs one).
// No instruction offset: it would move the LDS address as well.
__device__ __forceinline__ void copy_to_lds(u32x4 desc, uint32_t voffset, uint32_t lds_base)
{
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(desc), "{m0}"(lds_base)
                 : "memory");
}

// The same for 4 bytes per lane, landing at lds_base + 4 * lane.
__device__ __forceinline__ void copy_to_lds_b32(u32x4 desc, uint32_t voffset, uint32_t lds_base)
{
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(desc), "{m0}"(lds_base)
                 : "memory");
}

// LDS byte address of a __shared__ object (wave-uniform)
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p);
}

// s_waitcnt immediate that waits for vmcnt <= n only (6-bit count: bits 3:0
// and 15:14; expcnt and lgkmcnt fields at their maximum)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

}  // namespace miattn

// probes.hip -- machine probes for the measurement (libmiprobe.so): the
// quantities the tang paper's time floor is built from (§9.2 "From traffic to
// time": a dependent kernel's launch cost, a DRAM round trip, bytes over
// bandwidth), and the ceilings the attention kernels are compared with.
//
//   empty kernel       what one launch costs on a stream
//   pointer chase      one thread following a random chain through a buffer
//                      much larger than the last-level cache: DRAM latency
//   MFMA ceiling       every SIMD issuing independent 32x32x16 bf16 MFMAs on
//                      non-constant operands; the shader clock it runs at
//                      (shader-cycle counter against the 100 MHz reference)
//   read ceiling       a grid-stride streaming read of a large buffer
//
// None of these is part of the attention path; the bench loads this library
// beside libmiattn.so.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "miprobe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

__global__ void __launch_bounds__(64) empty_kernel() {}

// one wave follows i <- next[i], hops times, every lane at the same address;
// the index is kept in a vector register (else the compiler makes the chain
// scalar and it runs through the scalar cache), and the last index is stored
// so that the loads cannot be dropped
__global__ void __launch_bounds__(64) chase_kernel(const uint32_t *next, uint32_t start, int hops,
                                                   uint32_t *out)
{
    uint32_t i;
    asm volatile("v_mov_b32 %0, %1" : "=v"(i) : "s"(start));
    for (int h = 0; h < hops; ++h)
        i = __builtin_nontemporal_load(next + i);
    if (threadIdx.x == 0)
        out[0] = i;
}

// Four independent accumulators per wave, so consecutive MFMAs of a wave do
// not wait for each other. Lane 0 of each workgroup's first wave records the
// shader-cycle and reference-clock counters around the loop.
__global__ void __launch_bounds__(256) mfma_kernel(int iters, float *sink, unsigned long long *clk)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.25f + 0.001f * (float)((lane * 7 + e * 13) & 63));
        b[e] = (__bf16)(0.5f - 0.002f * (float)((lane * 5 + e * 3) & 63));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        s += c0[r] + c1[r] + c2[r] + c3[r];
    sink[blockIdx.x * 256 + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        clk[4 * blockIdx.x + 0] = t0;
        clk[4 * blockIdx.x + 1] = t1;
        clk[4 * blockIdx.x + 2] = r0;
        clk[4 * blockIdx.x + 3] = r1;
    }
}

// grid-stride read of n16 16-byte words; the XOR of everything read goes to
// sink (one word per wave) so that the loads are not dropped
__global__ void __launch_bounds__(256) read_kernel(const void *p, size_t n16, uint32_t *sink)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 *q = static_cast<const u32x4 *>(p);
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(q + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    acc ^= __shfl_xor(acc, 32, 64);
    acc ^= __shfl_xor(acc, 16, 64);
    acc ^= __shfl_xor(acc, 8, 64);
    acc ^= __shfl_xor(acc, 4, 64);
    acc ^= __shfl_xor(acc, 2, 64);
    acc ^= __shfl_xor(acc, 1, 64);
    if ((threadIdx.x & 63) == 0)
        sink[(size_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

int status(hipError_t e) { return e == hipSuccess ? 0 : (int)e; }

}  // namespace

extern "C" {

int probe_empty(int n_launches, hipStream_t stream)
{
    if (n_launches < 0)
        return -1;
    for (int i = 0; i < n_launches; ++i)
        hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
    return status(hipGetLastError());
}

int probe_chase(const uint32_t *next, size_t n_elems, uint32_t start, int hops, uint32_t *out,
                hipStream_t stream)
{
    if (next == nullptr || out == nullptr || hops < 0 || (size_t)start >= n_elems)
        return -1;
    hipLaunchKernelGGL(chase_kernel, dim3(1), dim3(64), 0, stream, next, start, hops, out);
    return status(hipGetLastError());
}

int probe_mfma(int blocks, int iters, float *sink, unsigned long long *clk, hipStream_t stream)
{
    if (blocks < 1 || iters < 0 || sink == nullptr || clk == nullptr)
        return -1;
    hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, iters, sink, clk);
    return status(hipGetLastError());
}

int probe_read(const void *buf, size_t bytes, int blocks, uint32_t *sink, hipStream_t stream)
{
    if (buf == nullptr || sink == nullptr || blocks < 1 || (bytes & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
        return -1;
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, buf, bytes / 16,
                       sink);
    return status(hipGetLastError());
}

}  // extern "C"

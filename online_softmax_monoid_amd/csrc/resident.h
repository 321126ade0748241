// resident.h -- how many workgroups of a kernel the current device holds at
// once, for persistent grids.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace miattn {

// Compute units times the kernel's occupancy; cached per device and per
// kernel. The kernel is a template argument, so every kernel has a cache of
// its own (keyed by its function type, kernels with one signature but
// different occupancies -- head dimensions, waves per SIMD -- would share
// one). 0 if the runtime cannot tell.
template <auto Kernel>
int resident_workgroups(int threads)
{
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    if (dev >= 0 && dev < kMaxDev) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0)
            return v;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, Kernel, threads, 0) != hipSuccess)
        return 0;
    const int v = cus * per_cu;
    if (v > 0 && dev >= 0 && dev < kMaxDev)
        cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

}  // namespace miattn

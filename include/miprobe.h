/*
 * miprobe.h -- C ABI of libmiprobe, the machine probes the benchmark reports
 * beside the attention kernels (not part of the attention path). They give
 * the terms of the time floor of the tang paper (muni.works/research/tang,
 * §9.2 "From traffic to time": a dependent kernel's launch cost, a DRAM
 * round trip, and bytes over bandwidth) and the ceilings the kernels are
 * compared with, measured on the machine at hand.
 *
 * All pointers are DEVICE pointers into caller-owned memory; nothing is
 * allocated; every call only enqueues work on `stream` and returns 0, or -1
 * for invalid arguments (nothing launched), or a positive hipError_t from
 * the launch. Timing is the caller's (events around the call).
 */
#ifndef MIPROBE_H
#define MIPROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__)
#define MIPROBE_API __attribute__((visibility("default")))
#else
#define MIPROBE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* n_launches >= 0 back-to-back launches of an empty kernel (one wave). */
MIPROBE_API int probe_empty(int n_launches, hipStream_t stream);

/*
 * One thread follows i <- next[i] `hops` times from `start` and stores the
 * final index to out[0]. next: uint32 [n_elems], every entry the chain
 * visits must be < n_elems (the caller builds the chain); start < n_elems.
 * With a random chain through a buffer several times the last-level cache,
 * the time per hop is the DRAM latency.
 */
MIPROBE_API int probe_chase(const uint32_t *next, size_t n_elems, uint32_t start, int hops,
                            uint32_t *out, hipStream_t stream);

/*
 * `blocks` workgroups of four waves; every wave issues iters * 32
 * v_mfma_f32_32x32x16_bf16 (32768 flop each) as four independent chains on
 * non-constant operands. sink: f32 [blocks * 256] (written, keeps the
 * results live); clk: u64 [blocks * 4] (written): per workgroup the
 * shader-cycle counter before and after the loop, then the 100 MHz
 * reference counter before and after, so cycles / (reference ticks / 1e8)
 * is the shader clock the MFMAs ran at.
 */
MIPROBE_API int probe_mfma(int blocks, int iters, float *sink, unsigned long long *clk,
                           hipStream_t stream);

/*
 * Grid-stride streaming read of `bytes` (a multiple of 16, buf 16-byte
 * aligned) by `blocks` workgroups of 256 threads; sink: u32 [blocks * 4]
 * (written).
 */
MIPROBE_API int probe_read(const void *buf, size_t bytes, int blocks, uint32_t *sink,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MIPROBE_H */

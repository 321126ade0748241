// launch.h -- internal interface between the C-ABI layer (api.cpp) and the
// kernel translation units. Arguments are already validated when these run.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace miattn {

struct FwdArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    uint16_t *o;
    float *lse;
    int B, Hq, Hkv, Sq, Sk;
    float scale;
    // sliding window: key j is visible to query i only if
    // j >= i + (Sk - Sq) - window; window < 0: no lower bound
    int window = -1;
    // score modifiers (at most one): soft cap s <- softcap * tanh(s / softcap)
    // of the scaled score (softcap > 0), or ALiBi s <- s - slope_h * |i + Sk - Sq - j|
    // with alibi[h] the slope of query head h (alibi != nullptr)
    float softcap = 0.f;
    const float *alibi = nullptr;
    // packed variable-length batch (cu_q != nullptr): q, o [Hq, total_q, d],
    // k, v [Hkv, total_k, d], lse [Hq, total_q]; sequence b's rows are
    // [cu_q[b], cu_q[b+1]) and keys [cu_k[b], cu_k[b+1]); Sq, Sk hold the
    // longest lengths
    const int *cu_q = nullptr;
    const int *cu_k = nullptr;
    int total_q = 0, total_k = 0;
};

struct DecodeArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    const int *lens;
    uint16_t *o;
    float *lse;
    float *part_acc;  // [B, Hq, splits, d]
    float *part_ml;   // [B, Hq, splits, 2]  (m in log2 units, l)
    int B, Hq, Hkv, S_cap, splits;
    float scale;
    // paged caches only (table == nullptr: contiguous [B, Hkv, S_cap, d]):
    // k, v are pools [num_pages, Hkv, page_size, d], table is [B, max_pages],
    // page_size = 1 << page_shift, S_cap = max_pages * page_size
    const int *table = nullptr;
    int max_pages = 0, num_pages = 0, page_shift = 0;
};

struct BwdArgs {
    const uint16_t *q, *k, *v, *o, *dout;
    const float *lse;
    uint16_t *dq, *dk, *dv;
    float *dsum;  // workspace: per row (D_i = dO_i . O_i, LSE_i log2 e), f32 [B, Hq, Sq, 2]
    int B, Hq, Hkv, Sq, Sk;
    float scale;
};

// Each returns hipSuccess or the launch error.
// prefill: the software-pipelined persistent kernel of prefill_kernel.h, one
// translation unit per head dimension
hipError_t launch_fwd_d64(const FwdArgs &a, bool causal, hipStream_t stream);
hipError_t launch_fwd_d128(const FwdArgs &a, bool causal, hipStream_t stream);
hipError_t launch_fwd_d256(const FwdArgs &a, bool causal, hipStream_t stream);
inline hipError_t launch_fwd(const FwdArgs &a, int d, bool causal, hipStream_t stream)
{
    switch (d) {
    case 64:
        return launch_fwd_d64(a, causal, stream);
    case 128:
        return launch_fwd_d128(a, causal, stream);
    case 256:
        return launch_fwd_d256(a, causal, stream);
    default:
        return hipErrorInvalidValue;
    }
}
hipError_t launch_decode(const DecodeArgs &a, int d, hipStream_t stream);
// The library's fixed decode scratch (decode.hip): its size in bytes, and its
// address on the current device (looked up on the first call per device).
size_t decode_scratch_bytes();
hipError_t decode_scratch(float **out);
// head dimensions 64 and 128: the backward kernels of backward.hip
hipError_t launch_bwd(const BwdArgs &a, int d, bool causal, hipStream_t stream);

}  // namespace miattn

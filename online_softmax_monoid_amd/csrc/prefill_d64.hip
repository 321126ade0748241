// prefill_d64.hip -- the prefill kernel of prefill_kernel.h at head dimension
// 64: four waves of 32 query rows (128 query rows per item), three workgroups
// per CU (three waves per SIMD: the softmax dominates at this head dimension,
// and a third wave per SIMD hides more of each item's start; measured 25%
// faster than two on items of a few tiles, the same on long ones).

#include "prefill_kernel.h"

namespace miattn {

hipError_t launch_fwd_d64(const FwdArgs &a, bool causal, hipStream_t stream)
{
    return launch_q64<64, 4, 3>(a, causal, stream);
}

}  // namespace miattn

// prefill_d256.hip -- the prefill kernel of prefill_kernel.h at head dimension
// 256: four waves of 32 query rows (one per SIMD: the f32
// accumulator alone takes 128 registers; 128 query rows per item).

#include "prefill_kernel.h"

namespace miattn {

hipError_t launch_fwd_d256(const FwdArgs &a, bool causal, hipStream_t stream)
{
    return launch_q64<256, 4, 1>(a, causal, stream);
}

}  // namespace miattn

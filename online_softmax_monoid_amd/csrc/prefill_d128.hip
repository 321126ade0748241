// prefill_d128.hip -- the prefill kernel of prefill_kernel.h at head dimension
// 128: eight waves of 32 query rows (two per SIMD, 256 query
// rows per item).

#include "prefill_kernel.h"

namespace miattn {

hipError_t launch_fwd_d128(const FwdArgs &a, bool causal, hipStream_t stream)
{
    return launch_q64<128, 8, 2>(a, causal, stream);
}

}  // namespace miattn

// pending.hip -- entry points whose kernels are not written yet report
// hipErrorNotSupported (surfaced as ATTN_EHIP with a message).
#include "common.hpp"

namespace attn {

hipError_t launch_fwd_materialized(float*, float*, float*, const float*, const Shape&,
                                   hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_bwd_materialized(float*, float*, float*, const float*, const float*,
                                   const float*, float*, const Shape&, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace attn

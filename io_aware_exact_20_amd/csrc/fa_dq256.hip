// The dQ pass at d = 256 (kernel in fa_dq16.hpp).  This translation unit
// is compiled without matrix-product results in VGPRs: the d = 256 kernel
// needs the AGPRs for its accumulators and scores.
#include "fa_dq16.hpp"

namespace fa {

hipError_t launch_bwd_dq16_256(Elem e, bool causal, bool dropout, const BwdArgs &a, hipStream_t stream) {
    switch (e) {
    case Elem::BF16: return launch_dq16_t<bf16, 256>(causal, dropout, a, stream);
    case Elem::F16: return launch_dq16_t<f16, 256>(causal, dropout, a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fa

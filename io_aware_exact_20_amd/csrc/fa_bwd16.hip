// Backward of fused exact attention for 16-bit inputs on gfx950: the dQ
// pass at d = 32, 64, 96 and 128 (the kernel is in fa_dq16.hpp; d = 256 is built in
// fa_dq256.hip, with other code-generation flags).
#include "fa_dq16.hpp"

namespace fa {

hipError_t launch_bwd_dq16(Elem e, int d, bool causal, bool dropout, const BwdArgs &a,
                           hipStream_t stream) {
    switch (e) {
    case Elem::BF16:
        return d == 32    ? launch_dq16_t<bf16, 32>(causal, dropout, a, stream)
               : d == 64  ? launch_dq16_t<bf16, 64>(causal, dropout, a, stream)
               : d == 96  ? launch_dq16_t<bf16, 96>(causal, dropout, a, stream)
               : d == 128 ? launch_dq16_t<bf16, 128>(causal, dropout, a, stream)
                          : launch_bwd_dq16_256(e, causal, dropout, a, stream);
    case Elem::F16:
        return d == 32    ? launch_dq16_t<f16, 32>(causal, dropout, a, stream)
               : d == 64  ? launch_dq16_t<f16, 64>(causal, dropout, a, stream)
               : d == 96  ? launch_dq16_t<f16, 96>(causal, dropout, a, stream)
               : d == 128 ? launch_dq16_t<f16, 128>(causal, dropout, a, stream)
                          : launch_bwd_dq16_256(e, causal, dropout, a, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace fa

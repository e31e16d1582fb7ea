// Reduced-precision kernels with f16 operands (one dtype per translation
// unit, so the two build in parallel).
#include "lowp.hpp"

namespace sgemm_impl {

hipError_t launch_lowp_f16(const LpProblem &p, hipStream_t stream) { return lp_launch_any<LpType::F16>(p, stream); }

}  // namespace sgemm_impl

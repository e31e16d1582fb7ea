// MFMA kernels for op(A) = A transposed, op(B) = B (one transpose pair per
// translation unit, so the four build in parallel).
#include "mfma.hpp"

namespace sgemm_impl {

hipError_t launch_mfma_tn(const Problem &p, hipStream_t stream)
{
    return launch_by_shape<true, false>(p, stream);
}

}  // namespace sgemm_impl

// MFMA kernels for op(A) = A transposed, op(B) = B (one transpose pair per
// translation unit, so the four build in parallel).
#include "mfma.hpp"

namespace sgemm_impl {

hipError_t launch_mfma_tn(const Problem &p, hipStream_t stream)
{
    return launch_by_shape<true, false>(p, stream);
}

hipError_t launch_mfma_sk_tn(const Problem &p, MfmaTile tile, float *ws, int grid, hipStream_t stream)
{
    return launch_sk_by_tile<true, false>(p, tile, ws, grid, stream);
}

}  // namespace sgemm_impl

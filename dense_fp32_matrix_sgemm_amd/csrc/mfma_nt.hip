// MFMA kernels for op(A) = A, op(B) = B transposed (one transpose pair per
// translation unit, so the four build in parallel).
#include "mfma.hpp"

namespace sgemm_impl {

hipError_t launch_mfma_nt(const Problem &p, hipStream_t stream)
{
    return launch_by_shape<false, true>(p, stream);
}

hipError_t launch_mfma_sk_nt(const Problem &p, MfmaTile tile, float *ws, int grid, hipStream_t stream)
{
    return launch_sk_by_tile<false, true>(p, tile, ws, grid, stream);
}

}  // namespace sgemm_impl

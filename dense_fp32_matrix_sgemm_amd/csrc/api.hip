// C ABI entry point: host checks, device check, variant dispatch, launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "gemm.hpp"
#include "sgemm.h"

namespace {

// Per-device cache: 0 = not yet asked, -1 = not a gfx950, otherwise the
// device's compute-unit count. Written once per device; racing writers store
// the same value.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_cus[kMaxDevices];

// Compute units of the current device if it is a gfx950, else 0.
int current_gfx950_cus()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev >= kMaxDevices) return 0;
    int state = g_device_cus[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
        // gcnArchName reads like "gfx950:sramecc+:xnack-".
        const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                        (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
        state = ok && prop.multiProcessorCount > 0 ? prop.multiProcessorCount : -1;
        g_device_cus[dev].store(state, std::memory_order_release);
    }
    return state > 0 ? state : 0;
}

}  // namespace

extern "C" int sgemm(int M, int N, int K, const float *A, int lda, const float *B, int ldb, float *C, int ldc,
                     void *stream, int variant)
{
    const int rc = sgemm_check_args(M, N, K, A, lda, B, ldb, C, ldc, variant);
    if (rc != SGEMM_OK) return rc;
    if (M == 0 || N == 0) return SGEMM_OK;
    const int cus = current_gfx950_cus();
    if (cus == 0) return SGEMM_ERR_DEVICE;

    const sgemm_impl::Problem p{A, B, C, lda, ldb, ldc, M, N, K, cus};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (variant == SGEMM_BEST) variant = sgemm_best_variant(M, N, K);

    hipError_t err;
    switch (variant) {
    case SGEMM_NAIVE: err = sgemm_impl::launch_naive(p, s); break;
    case SGEMM_TILED: err = sgemm_impl::launch_tiled(p, s); break;
    case SGEMM_REGBLOCK: err = sgemm_impl::launch_regblock(p, s); break;
    case SGEMM_MFMA: err = sgemm_impl::launch_mfma(p, s); break;
    default: return SGEMM_ERR_VARIANT;
    }
    return err == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

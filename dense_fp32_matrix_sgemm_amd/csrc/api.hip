// C ABI entry point: host checks, device check, variant dispatch, launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "gemm.hpp"
#include "sgemm.h"

namespace {

// Per-device answer to "is this a gfx950?": 0 = not yet asked, 1 = yes,
// 2 = no. Written once per device; racing writers store the same value.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

bool current_device_is_gfx950()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
    if (dev >= kMaxDevices) return false;
    int state = g_arch_ok[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
        // gcnArchName reads like "gfx950:sramecc+:xnack-".
        const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                        (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
        state = ok ? 1 : 2;
        g_arch_ok[dev].store(state, std::memory_order_release);
    }
    return state == 1;
}

}  // namespace

extern "C" int sgemm(int M, int N, int K, const float *A, int lda, const float *B, int ldb, float *C, int ldc,
                     void *stream, int variant)
{
    const int rc = sgemm_check_args(M, N, K, A, lda, B, ldb, C, ldc, variant);
    if (rc != SGEMM_OK) return rc;
    if (M == 0 || N == 0) return SGEMM_OK;
    if (!current_device_is_gfx950()) return SGEMM_ERR_DEVICE;

    const sgemm_impl::Problem p{A, B, C, lda, ldb, ldc, M, N, K};
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

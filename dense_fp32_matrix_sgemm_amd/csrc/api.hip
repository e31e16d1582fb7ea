// C ABI entry point: host checks, device check, variant dispatch, launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>
#include <cstring>

#include "gemm.hpp"
#include "select.hpp"
#include "sgemm.h"

namespace {

// Per-device cache: 0 = not yet asked, -1 = not a gfx950, otherwise the
// device's compute-unit count. Written once per device; racing writers store
// the same value.
std::atomic<int> g_device_cus[sgemm_impl::kMaxDevices];

}  // namespace

// Compute units of the current device if it is a gfx950, else 0.
int sgemm_impl::current_gfx950_cus()
{
    using sgemm_impl::kMaxDevices;
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

namespace {
using sgemm_impl::current_gfx950_cus;

hipError_t launch_mfma(const sgemm_impl::Problem &p, hipStream_t s)
{
    if (p.ta) return p.tb ? sgemm_impl::launch_mfma_tt(p, s) : sgemm_impl::launch_mfma_tn(p, s);
    return p.tb ? sgemm_impl::launch_mfma_nt(p, s) : sgemm_impl::launch_mfma_nn(p, s);
}

hipError_t launch_mfma_sk(const sgemm_impl::Problem &p, sgemm_impl::MfmaTile tile, float *ws, int grid, hipStream_t s)
{
    if (p.ta)
        return p.tb ? sgemm_impl::launch_mfma_sk_tt(p, tile, ws, grid, s) : sgemm_impl::launch_mfma_sk_tn(p, tile, ws, grid, s);
    return p.tb ? sgemm_impl::launch_mfma_sk_nt(p, tile, ws, grid, s) : sgemm_impl::launch_mfma_sk_nn(p, tile, ws, grid, s);
}

}  // namespace

extern "C" int sgemm_ex_ws(int transA, int transB, int M, int N, int K, float alpha, const float *A, int lda,
                           const float *B, int ldb, float beta, float *C, int ldc, void *workspace,
                           std::size_t workspace_bytes, void *stream, int variant)
{
    const int rc = sgemm_ex_ws_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                                          workspace_bytes, variant);
    if (rc != SGEMM_OK) return rc;
    const bool product = M > 0 && N > 0 && K > 0 && alpha != 0.0f;
    const int v = variant == SGEMM_BEST ? sgemm_best_variant(M, N, K) : variant;
    // The adding kernel reads the partial tiles with 16-byte loads, so a
    // workspace that is not 16-byte aligned is not used.
    const bool ws_usable =
        workspace != nullptr && workspace_bytes > 0 && reinterpret_cast<std::uintptr_t>(workspace) % 16 == 0;
    if (product && v == SGEMM_MFMA && ws_usable) {
        const int cus = current_gfx950_cus();
        if (cus == 0) return SGEMM_ERR_DEVICE;
        const std::size_t need = sgemm_ex_workspace_size(transA, transB, M, N, K, cus);
        if (need > 0 && need <= workspace_bytes) {
            const sgemm_impl::SplitChoice c = sgemm_impl::choose_split(M, N, K, cus);
            const sgemm_impl::Problem p{A,     B,    C,   lda, ldb, ldc, M, N, K, cus, transA == SGEMM_OP_T,
                                        transB == SGEMM_OP_T, alpha, beta, c.tile};
            const hipError_t err =
                launch_mfma_sk(p, c.tile, static_cast<float *>(workspace), c.grid, static_cast<hipStream_t>(stream));
            return err == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
        }
    }
    return sgemm_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant);
}

extern "C" int sgemm_ex(int transA, int transB, int M, int N, int K, float alpha, const float *A, int lda,
                        const float *B, int ldb, float beta, float *C, int ldc, void *stream, int variant)
{
    const int rc = sgemm_ex_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant);
    if (rc != SGEMM_OK) return rc;
    if (M == 0 || N == 0) return SGEMM_OK;
    const bool product = K > 0 && alpha != 0.0f;
    if (!product && beta == 1.0f) return SGEMM_OK;  // C = 1 * C: nothing to do
    const int cus = current_gfx950_cus();
    if (cus == 0) return SGEMM_ERR_DEVICE;

    const sgemm_impl::Problem p{A,     B,    C,   lda, ldb, ldc, M, N, K, cus, transA == SGEMM_OP_T, transB == SGEMM_OP_T,
                                alpha, beta, sgemm_impl::choose_mfma_tile(M, N, K, cus)};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (variant == SGEMM_BEST) variant = sgemm_best_variant(M, N, K);

    hipError_t err;
    if (!product) {
        err = sgemm_impl::launch_scale(p, s);
    } else {
        switch (variant) {
        case SGEMM_NAIVE: err = sgemm_impl::launch_naive(p, s); break;
        case SGEMM_TILED: err = sgemm_impl::launch_tiled(p, 0, s); break;
        case SGEMM_TILED_T8: err = sgemm_impl::launch_tiled(p, 8, s); break;
        case SGEMM_TILED_T16: err = sgemm_impl::launch_tiled(p, 16, s); break;
        case SGEMM_TILED_T32: err = sgemm_impl::launch_tiled(p, 32, s); break;
        case SGEMM_REGBLOCK: err = sgemm_impl::launch_regblock(p, s); break;
        case SGEMM_MFMA: err = launch_mfma(p, s); break;
        default: return SGEMM_ERR_VARIANT;
        }
    }
    return err == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

extern "C" int sgemm_lp(int dtype, int transA, int transB, int M, int N, int K, float alpha, const void *A, int lda,
                        const void *B, int ldb, float beta, float *C, int ldc, void *stream)
{
    const int rc = sgemm_lp_check_args(dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
    if (rc != SGEMM_OK) return rc;
    if (M == 0 || N == 0) return SGEMM_OK;
    const bool product = K > 0 && alpha != 0.0f;
    if (!product && beta == 1.0f) return SGEMM_OK;
    const int cus = current_gfx950_cus();
    if (cus == 0) return SGEMM_ERR_DEVICE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (!product) {
        const sgemm_impl::Problem p{nullptr, nullptr, C, 1, 1, ldc, M, N, K, cus, false, false, alpha, beta,
                                    sgemm_impl::MfmaTile::Big};
        err = sgemm_impl::launch_scale(p, s);
    } else {
        const sgemm_impl::LpProblem p{static_cast<const std::uint16_t *>(A), static_cast<const std::uint16_t *>(B),
                                      C, lda, ldb, ldc, M, N, K, cus, transA == SGEMM_OP_T, transB == SGEMM_OP_T,
                                      alpha, beta};
        err = dtype == SGEMM_LP_BF16 ? sgemm_impl::launch_lowp_bf16(p, s) : sgemm_impl::launch_lowp_f16(p, s);
    }
    return err == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

extern "C" int sgemm(int M, int N, int K, const float *A, int lda, const float *B, int ldb, float *C, int ldc,
                     void *stream, int variant)
{
    return sgemm_ex(SGEMM_OP_N, SGEMM_OP_N, M, N, K, 1.0f, A, lda, B, ldb, 0.0f, C, ldc, stream, variant);
}

// sgemm_ex_noalloc: the general product with the split schedule's scratch in
// a static device buffer of the library's own, for callers that cannot
// allocate device memory (code under stream capture, tight loops, harnesses
// that forbid hipMalloc).
//
// The buffer below is a file-scope device array: each GPU the library runs
// on holds its own copy, at its own address, from when the library's code is
// loaded on that GPU until the process ends. In host code the array's name
// is only a host-side stand-in, never a device address: the address a kernel
// may use is looked up per device with hipGetSymbolAddress, once, on the
// entry point's first call on that device (with that device current), and
// only that address is ever passed on.
//
// Every call on one GPU shares that GPU's buffer. The split schedule writes
// each partial tile before the adding kernel reads it, so nothing in the
// buffer has to start at zero and what an earlier call left there is never
// read; but calls whose kernels can overlap on one GPU (different streams
// without an ordering between them) race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "gemm.hpp"
#include "select.hpp"
#include "sgemm.h"

namespace {

static_assert(sgemm_impl::kNoallocScratchBytes % 256 == 0, "whole 256-byte units");

static __device__ __align__(256) float scratch[sgemm_impl::kNoallocScratchBytes / sizeof(float)];

// Per-device device address of `scratch` (nullptr until looked up).
std::atomic<float *> g_scratch[sgemm_impl::kMaxDevices];
std::mutex g_scratch_mutex;

// The current device's address of `scratch`, looked up on first use; nullptr
// if the device cannot be named or the lookup fails.
float *scratch_of_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= sgemm_impl::kMaxDevices) return nullptr;
    float *ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (ptr != nullptr) return ptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return nullptr;
        ptr = static_cast<float *>(addr);
        g_scratch[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

}  // namespace

extern "C" int sgemm_ex_noalloc(int transA, int transB, int M, int N, int K, float alpha, const float *A, int lda,
                                const float *B, int ldb, float beta, float *C, int ldc, void *stream, int variant)
{
    const int rc = sgemm_ex_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant);
    if (rc != SGEMM_OK) return rc;
    const bool product = M > 0 && N > 0 && K > 0 && alpha != 0.0f;
    const int v = variant == SGEMM_BEST ? sgemm_best_variant(M, N, K) : variant;
    if (!product || v != SGEMM_MFMA)
        return sgemm_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant);
    const int cus = sgemm_impl::current_gfx950_cus();
    if (cus == 0) return SGEMM_ERR_DEVICE;
    const std::size_t need = sgemm_ex_workspace_size(transA, transB, M, N, K, cus);
    if (need > sgemm_impl::kNoallocScratchBytes) return SGEMM_ERR_SCRATCH;
    if (need == 0)  // whole tiles: no scratch
        return sgemm_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant);
    float *ws = scratch_of_current_device();
    if (ws == nullptr) return SGEMM_ERR_DEVICE;
    return sgemm_ex_ws(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ws,
                       sgemm_impl::kNoallocScratchBytes, stream, variant);
}

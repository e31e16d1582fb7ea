// C = beta * C over the M x N window: the whole of C = alpha * op(A) * op(B)
// + beta * C when the product term vanishes (K == 0 or alpha == 0), in which
// case A and B are not read. beta == 0 stores zeros without reading C, so
// NaN or Inf already in C does not survive (the BLAS convention).
#include "gemm.hpp"

namespace sgemm_impl {
namespace {

constexpr int kThreads = 256;
constexpr unsigned kMaxGridX = 1024;

__global__ __launch_bounds__(kThreads) void scale_kernel(float *C, std::int64_t ldc, int M, int N, float beta)
{
    for (std::int64_t row = blockIdx.y; row < M; row += gridDim.y) {
        float *c = C + row * ldc;
        for (std::int64_t col = std::int64_t(blockIdx.x) * kThreads + threadIdx.x; col < N;
             col += std::int64_t(gridDim.x) * kThreads)
            c[col] = beta != 0.0f ? beta * c[col] : 0.0f;
    }
}

}  // namespace

hipError_t launch_scale(const Problem &p, hipStream_t stream)
{
    const unsigned long long cols = (static_cast<unsigned long long>(p.N) + kThreads - 1) / kThreads;
    const unsigned gx = cols < kMaxGridX ? unsigned(cols) : kMaxGridX;
    const unsigned gy = unsigned(p.M) < kMaxGridY ? unsigned(p.M) : kMaxGridY;
    float *C = p.C;
    std::int64_t ldc = p.ldc;
    int M = p.M, N = p.N;
    float beta = p.beta;
    void *args[] = {&C, &ldc, &M, &N, &beta};
    return hipLaunchKernel(reinterpret_cast<const void *>(&scale_kernel), dim3(gx, gy), dim3(kThreads), args, 0,
                           stream);
}

}  // namespace sgemm_impl

// Rung 1: one work-item per element of C, operands read straight from global
// memory ("Matrix Multiplication -- Naive to Tiled", section 02; "Naive GEMM vs
// Tiled GEMM", naive kernel).
//
// Work-group 64 x 4: each wave64 owns 64 consecutive columns of one row, so
// its 64 loads of B per k step are one contiguous 256-byte row segment and its
// load of A is a single address shared by the whole wave.
#include "gemm.hpp"

namespace sgemm_impl {
namespace {

constexpr int kBX = 64;  // columns per work-group (one wave)
constexpr int kBY = 4;   // rows per work-group (four waves)

__global__ __launch_bounds__(kBX *kBY) void naive_kernel(Problem p)
{
    const int col = blockIdx.x * kBX + threadIdx.x;
    if (col >= p.N) return;
    for (std::int64_t row = std::int64_t(blockIdx.y) * kBY + threadIdx.y; row < p.M;
         row += std::int64_t(gridDim.y) * kBY) {
        const float *a = p.A + row * p.lda;
        const float *b = p.B + col;
        float acc = 0.0f;
        for (int k = 0; k < p.K; ++k) acc = __builtin_fmaf(a[k], b[std::int64_t(k) * p.ldb], acc);
        p.C[row * p.ldc + col] = acc;
    }
}

}  // namespace

hipError_t launch_naive(const Problem &p, hipStream_t stream)
{
    const unsigned gx = unsigned((p.N + kBX - 1) / kBX);
    const unsigned long long rows = (static_cast<unsigned long long>(p.M) + kBY - 1) / kBY;
    const unsigned gy = rows < kMaxGridY ? unsigned(rows) : kMaxGridY;
    Problem arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&naive_kernel), dim3(gx, gy), dim3(kBX, kBY), args, 0,
                           stream);
}

}  // namespace sgemm_impl

// Rung 1: one work-item per element of C, operands read straight from global
// memory ("Matrix Multiplication -- Naive to Tiled", section 02; "Naive GEMM vs
// Tiled GEMM", naive kernel), extended to C = alpha * op(A) * op(B) + beta * C.
//
// Work-group 64 x 4: each wave64 owns 64 consecutive columns of one row, so
// its load of op(A) per k step is a single address shared by the whole wave,
// and its 64 loads of op(B) are one contiguous 256-byte row segment when B is
// as given (64 rows ldb apart when B is transposed: this rung does not
// restage).
#include "gemm.hpp"
#include "tile_io.hpp"

namespace sgemm_impl {
namespace {

constexpr int kBX = 64;  // columns per work-group (one wave)
constexpr int kBY = 4;   // rows per work-group (four waves)

template <bool TA, bool TB>
__global__ __launch_bounds__(kBX *kBY) void naive_kernel(Problem p)
{
    const int col = blockIdx.x * kBX + threadIdx.x;
    if (col >= p.N) return;
    // Strides between consecutive k of op(A)'s row and of op(B)'s column.
    const std::int64_t sa = TA ? p.lda : 1, sb = TB ? 1 : p.ldb;
    for (std::int64_t row = std::int64_t(blockIdx.y) * kBY + threadIdx.y; row < p.M;
         row += std::int64_t(gridDim.y) * kBY) {
        const float *a = TA ? p.A + row : p.A + row * p.lda;
        const float *b = TB ? p.B + std::int64_t(col) * p.ldb : p.B + col;
        float acc = 0.0f;
        for (int k = 0; k < p.K; ++k) acc = __builtin_fmaf(a[k * sa], b[k * sb], acc);
        float *c = p.C + row * p.ldc + col;
        *c = p.beta != 0.0f ? axpby(p.alpha, acc, p.beta, *c) : p.alpha * acc;
    }
}

template <bool TA, bool TB>
hipError_t launch(const Problem &p, hipStream_t stream)
{
    const unsigned gx = unsigned((p.N + kBX - 1) / kBX);
    const unsigned long long rows = (static_cast<unsigned long long>(p.M) + kBY - 1) / kBY;
    const unsigned gy = rows < kMaxGridY ? unsigned(rows) : kMaxGridY;
    Problem arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&naive_kernel<TA, TB>), dim3(gx, gy), dim3(kBX, kBY),
                           args, 0, stream);
}

}  // namespace

hipError_t launch_naive(const Problem &p, hipStream_t stream)
{
    if (p.ta) return p.tb ? launch<true, true>(p, stream) : launch<true, false>(p, stream);
    return p.tb ? launch<false, true>(p, stream) : launch<false, false>(p, stream);
}

}  // namespace sgemm_impl

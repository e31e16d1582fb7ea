// Rung 2: LDS tiling with boundary guards ("Matrix Multiplication -- Naive to
// Tiled", sections 04-05; "Shared Memory Tiling for Matrix Multiplication",
// tiling, barriers and traps).
//
// A T x T work-group owns a T x T tile of C. For each K step of T it stages a
// T x T tile of A and of B in LDS (elements outside the matrices read as 0,
// which is what makes ragged M, N and K correct), waits at a barrier, does T
// multiply-adds per work-item from LDS, and waits again before the next step
// overwrites the tiles.
//
// With T = 16 a wave64 covers four rows of the tile. The four rows read four
// different words of As in the same instruction, so As rows are padded by one
// word to put them in different banks; the B tile is read as one contiguous
// row segment (a broadcast across the four rows) and needs no padding.
#include "gemm.hpp"

namespace sgemm_impl {
namespace {

constexpr int kT = 16;

__global__ __launch_bounds__(kT *kT) void tiled_kernel(Problem p)
{
    __shared__ float As[kT][kT + 1];
    __shared__ float Bs[kT][kT];

    const int tx = threadIdx.x, ty = threadIdx.y;
    const int col = blockIdx.x * kT + tx;

    for (std::int64_t row0 = std::int64_t(blockIdx.y) * kT; row0 < p.M; row0 += std::int64_t(gridDim.y) * kT) {
        const std::int64_t row = row0 + ty;
        float acc = 0.0f;
        for (int k0 = 0; k0 < p.K; k0 += kT) {
            const int ka = k0 + tx;  // column of A this work-item stages
            const int kb = k0 + ty;  // row of B this work-item stages
            As[ty][tx] = (row < p.M && ka < p.K) ? p.A[row * p.lda + ka] : 0.0f;
            Bs[ty][tx] = (kb < p.K && col < p.N) ? p.B[std::int64_t(kb) * p.ldb + col] : 0.0f;
            __syncthreads();  // tiles complete before anyone reads them
#pragma unroll
            for (int k = 0; k < kT; ++k) acc = __builtin_fmaf(As[ty][k], Bs[k][tx], acc);
            __syncthreads();  // everyone done reading before the next overwrite
        }
        if (row < p.M && col < p.N) p.C[row * p.ldc + col] = acc;
    }
}

}  // namespace

hipError_t launch_tiled(const Problem &p, hipStream_t stream)
{
    const unsigned gx = unsigned((p.N + kT - 1) / kT);
    const unsigned long long rows = (static_cast<unsigned long long>(p.M) + kT - 1) / kT;
    const unsigned gy = rows < kMaxGridY ? unsigned(rows) : kMaxGridY;
    Problem arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&tiled_kernel), dim3(gx, gy), dim3(kT, kT), args, 0,
                           stream);
}

}  // namespace sgemm_impl

// Rung 2: LDS tiling with boundary guards ("Matrix Multiplication -- Naive to
// Tiled", sections 04-05; "Shared Memory Tiling for Matrix Multiplication",
// tiling, barriers and traps), extended to C = alpha * op(A) * op(B) + beta * C.
//
// A T x T work-group owns a T x T tile of C. For each K step of T it stages a
// T x T tile of op(A) and of op(B) in LDS (elements outside the matrices read
// as 0, which is what makes ragged M, N and K correct), waits at a barrier,
// does T multiply-adds per work-item from LDS, and waits again before the
// next step overwrites the tiles.
//
// Staging reads consecutive addresses across the 16 work-items of a tile row
// whatever the storage order: an operand stored transposed is read along its
// stored rows and written transposed into LDS.
//
// With T = 16 a wave64 covers four rows of the tile. The four rows read four
// different words of As in the same instruction, so As rows are padded by one
// word to put them in different banks (the padding also spreads the
// transposed writes); Bs is read as one contiguous row segment (a broadcast
// across the four rows) and is padded only when it is written transposed.
#include "gemm.hpp"
#include "tile_io.hpp"

namespace sgemm_impl {
namespace {

constexpr int kT = 16;

template <bool TA, bool TB>
__global__ __launch_bounds__(kT *kT) void tiled_kernel(Problem p)
{
    __shared__ float As[kT][kT + 1];                 // As[i][k] = op(A)[row0 + i][k0 + k]
    __shared__ float Bs[kT][kT + (TB ? 1 : 0)];      // Bs[k][j] = op(B)[k0 + k][col0 + j]

    const int tx = threadIdx.x, ty = threadIdx.y;
    const int col0 = blockIdx.x * kT;
    const int col = col0 + tx;

    for (std::int64_t row0 = std::int64_t(blockIdx.y) * kT; row0 < p.M; row0 += std::int64_t(gridDim.y) * kT) {
        const std::int64_t row = row0 + ty;
        float acc = 0.0f;
        for (int k0 = 0; k0 < p.K; k0 += kT) {
            if constexpr (!TA) {  // A stored M x K: work-item reads A[row][k0 + tx]
                As[ty][tx] = (row < p.M && k0 + tx < p.K) ? p.A[row * p.lda + k0 + tx] : 0.0f;
            } else {  // A stored K x M: work-item reads A[k0 + ty][row0 + tx]
                As[tx][ty] = (k0 + ty < p.K && row0 + tx < p.M) ? p.A[std::int64_t(k0 + ty) * p.lda + row0 + tx] : 0.0f;
            }
            if constexpr (!TB) {  // B stored K x N: work-item reads B[k0 + ty][col]
                Bs[ty][tx] = (k0 + ty < p.K && col < p.N) ? p.B[std::int64_t(k0 + ty) * p.ldb + col] : 0.0f;
            } else {  // B stored N x K: work-item reads B[col0 + ty][k0 + tx]
                Bs[tx][ty] = (col0 + ty < p.N && k0 + tx < p.K) ? p.B[std::int64_t(col0 + ty) * p.ldb + k0 + tx] : 0.0f;
            }
            __syncthreads();  // tiles complete before anyone reads them
#pragma unroll
            for (int k = 0; k < kT; ++k) acc = __builtin_fmaf(As[ty][k], Bs[k][tx], acc);
            __syncthreads();  // everyone done reading before the next overwrite
        }
        if (row < p.M && col < p.N) {
            float *c = p.C + row * p.ldc + col;
            *c = p.beta != 0.0f ? axpby(p.alpha, acc, p.beta, *c) : p.alpha * acc;
        }
    }
}

template <bool TA, bool TB>
hipError_t launch(const Problem &p, hipStream_t stream)
{
    const unsigned gx = unsigned((p.N + kT - 1) / kT);
    const unsigned long long rows = (static_cast<unsigned long long>(p.M) + kT - 1) / kT;
    const unsigned gy = rows < kMaxGridY ? unsigned(rows) : kMaxGridY;
    Problem arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&tiled_kernel<TA, TB>), dim3(gx, gy), dim3(kT, kT), args,
                           0, stream);
}

}  // namespace

hipError_t launch_tiled(const Problem &p, hipStream_t stream)
{
    if (p.ta) return p.tb ? launch<true, true>(p, stream) : launch<true, false>(p, stream);
    return p.tb ? launch<false, true>(p, stream) : launch<false, false>(p, stream);
}

}  // namespace sgemm_impl

// Rung 2: LDS tiling with boundary guards ("Matrix Multiplication -- Naive to
// Tiled", sections 04-05 and exercise 2; "Shared Memory Tiling for
// Matrix Multiplication", tiling, barriers and traps; "Naive GEMM vs Tiled
// GEMM", the tiled kernel with 32 x 32 tiles), extended to
// C = alpha * op(A) * op(B) + beta * C.
//
// A T x T work-group owns a T x T tile of C, T in {8, 16, 32}. For each K step
// of T it stages a T x T tile of op(A) and of op(B) in LDS (elements outside
// the matrices read as 0, which is what makes ragged M, N and K correct),
// waits at a barrier, does T multiply-adds per work-item from LDS, and waits
// again before the next step overwrites the tiles.
//
// Staging reads consecutive addresses across the T work-items of a tile row
// whatever the storage order: an operand stored transposed is read along its
// stored rows and written transposed into LDS.
//
// A wave64 covers 64 / T rows of the tile (8, 4 or 2). Those rows read
// different words of As in the same instruction, so As rows are padded by one
// word to put them in different banks (the padding also spreads the
// transposed writes); Bs is read as one contiguous row segment (a broadcast
// across the rows) and is padded only when it is written transposed.
//
// Work-groups are numbered along one dimension and mapped to tiles the way
// the matrix-core rung maps them: each of the eight XCDs (each with its own
// L2) takes one contiguous run of tiles, walked in bands of 8 tile rows,
// column by column, so that the work-groups resident on one XCD at a time
// share a few rows of A and columns of B in its L2. With the pages' plain
// two-dimensional grid the tiles resident on an XCD lay along whole tile
// rows, and nearly every tile load left the L2: at 4096^3 and T = 16 the L2s
// fetched 34.4 GB from the fabric, 2 N^3 * 4 / T, every tile load missing.
// Bands of 2, 4, 8, 16, 32 and 64 tile rows fetched 9.3, 4.4, 2.3, 6.7, 17.9
// and 18.1 GB (T = 32: 4.8, 3.2, 3.1, 4.8, 8.8 and 8.9 GB), against 2.9 GB
// for the naive rung, with launch times within 2% of each other.
#include "gemm.hpp"
#include "tile_io.hpp"

namespace sgemm_impl {
namespace {

// Tile rows per band of the tile order.
#ifndef SGEMM_TILED_GROUP_M
#define SGEMM_TILED_GROUP_M 8
#endif
template <int T>
constexpr int kGroupM = SGEMM_TILED_GROUP_M;

template <int T, bool TA, bool TB>
__global__ __launch_bounds__(T *T) void tiled_kernel(Problem p, int tiles_m)
{
    __shared__ float As[T][T + 1];                 // As[i][k] = op(A)[row0 + i][k0 + k]
    __shared__ float Bs[T][T + (TB ? 1 : 0)];      // Bs[k][j] = op(B)[k0 + k][col0 + j]

    int tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, kGroupM<T>, tm, tn);
    const int tx = threadIdx.x, ty = threadIdx.y;
    const std::int64_t row0 = std::int64_t(tm) * T;
    const int col0 = tn * T;
    const std::int64_t row = row0 + ty;
    const int col = col0 + tx;

    float acc = 0.0f;
    for (int k0 = 0; k0 < p.K; k0 += T) {
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
        for (int k = 0; k < T; ++k) acc = __builtin_fmaf(As[ty][k], Bs[k][tx], acc);
        __syncthreads();  // everyone done reading before the next overwrite
    }
    if (row < p.M && col < p.N) {
        float *c = p.C + row * p.ldc + col;
        *c = p.beta != 0.0f ? axpby(p.alpha, acc, p.beta, *c) : p.alpha * acc;
    }
}

// One launch per band of at most 2^20 tiles (2^30 work-items at T = 32).
template <int T, bool TA, bool TB>
hipError_t launch(const Problem &p, hipStream_t stream)
{
    return for_each_band<T, T>(
        p,
        [&](const Problem &q, int tiles_m, int tiles_n) {
            Problem arg = q;
            int tm_arg = tiles_m;
            void *args[] = {&arg, &tm_arg};
            return hipLaunchKernel(reinterpret_cast<const void *>(&tiled_kernel<T, TA, TB>),
                                   dim3(unsigned(tiles_m) * unsigned(tiles_n)), dim3(T, T), args, 0, stream);
        },
        std::int64_t(1) << 20);
}

template <int T>
hipError_t launch_t(const Problem &p, hipStream_t stream)
{
    if (p.ta) return p.tb ? launch<T, true, true>(p, stream) : launch<T, true, false>(p, stream);
    return p.tb ? launch<T, false, true>(p, stream) : launch<T, false, false>(p, stream);
}

}  // namespace

int tiled_tile_size(int M, int N)
{
    // Sweep of T = 8, 16 and 32 on MI355X (median launch times, microseconds):
    //   128^3 9.0 / 7.8 / 9.9;  1024^3 159 / 142 / 137;  2048^3 1265 / 1052 /
    //   1049;  4096^3 10343 / 8200 / 8494;  3001 x 2047 x 4093 3988 / 3092 /
    //   3384.
    // Every T runs at 13-17 TFLOP/s: each multiply-add takes two LDS reads
    // whatever T is, so the rung is bound by LDS bandwidth and T moves it
    // little. 8 x 8 tiles (one wave per work-group) always lose; 32 x 32 wins
    // by 4% where C holds 2-8 of its tiles per compute unit, and 16 x 16 by
    // 4-9% on larger products and at 128^3.
    const std::int64_t tiles32 = ((std::int64_t(M) + 31) / 32) * ((std::int64_t(N) + 31) / 32);
    return tiles32 >= 2 * 256 && tiles32 <= 8 * 256 ? 32 : 16;
}

hipError_t launch_tiled(const Problem &p, int T, hipStream_t stream)
{
    if (T == 0) T = tiled_tile_size(p.M, p.N);
    switch (T) {
    case 8: return launch_t<8>(p, stream);
    case 16: return launch_t<16>(p, stream);
    default: return launch_t<32>(p, stream);
    }
}

}  // namespace sgemm_impl

// Internal interface between the C ABI's dispatcher and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tiles.hpp"

namespace sgemm_impl {

// One product C = alpha * op(A) * op(B) + beta * C, row-major, leading
// dimensions in elements. op(A) is M x K: A itself (stored M x K) or, with
// ta, the transpose of A (stored K x M); op(B) is K x N: B (stored K x N) or,
// with tb, the transpose of B (stored N x K). Offsets are formed in 64 bits
// so that any int-sized problem indexes correctly.
struct Problem {
    const float *A;
    const float *B;
    float *C;
    std::int64_t lda, ldb, ldc;
    int M, N, K;
    int cus;  // compute units of the device (for the choice of tile size)
    bool ta, tb;
    float alpha, beta;  // C is read only when beta != 0
    MfmaTile tile;      // interior tile shape of the matrix-core variant
};

// Each launcher enqueues the variant's kernel(s) on `stream` and returns the
// launch status; the problem has already been validated and has work to do:
// M > 0, N > 0, K > 0 and alpha != 0 (the other cases only scale C).
hipError_t launch_naive(const Problem &p, hipStream_t stream);
// The tiled rung with T x T tiles, T in {8, 16, 32}; T = 0 takes
// tiled_tile_size(M, N), the tile the rung picks for the shape.
hipError_t launch_tiled(const Problem &p, int T, hipStream_t stream);
int tiled_tile_size(int M, int N);
hipError_t launch_regblock(const Problem &p, hipStream_t stream);
hipError_t launch_mfma_nn(const Problem &p, hipStream_t stream);  // one per transpose pair
hipError_t launch_mfma_nt(const Problem &p, hipStream_t stream);
hipError_t launch_mfma_tn(const Problem &p, hipStream_t stream);
hipError_t launch_mfma_tt(const Problem &p, hipStream_t stream);
// The matrix-core variant on the split schedule (mfma.hpp): `grid`
// work-groups with `tile` shapes, partial tiles in `ws` (at least
// split_workspace_bytes(tile, grid) bytes, select.hpp).
hipError_t launch_mfma_sk_nn(const Problem &p, MfmaTile tile, float *ws, int grid, hipStream_t stream);
hipError_t launch_mfma_sk_nt(const Problem &p, MfmaTile tile, float *ws, int grid, hipStream_t stream);
hipError_t launch_mfma_sk_tn(const Problem &p, MfmaTile tile, float *ws, int grid, hipStream_t stream);
hipError_t launch_mfma_sk_tt(const Problem &p, MfmaTile tile, float *ws, int grid, hipStream_t stream);
// C = beta * C over the M x N window (zeros, without reading C, when beta is
// 0): the whole product when K == 0 or alpha == 0.
hipError_t launch_scale(const Problem &p, hipStream_t stream);

// First element of op(A)'s row r (A's column r when transposed) and of
// op(B)'s column c (B's row c when transposed).
__host__ __device__ inline const float *a_row_start(const Problem &p, std::int64_t r) { return p.ta ? p.A + r : p.A + r * p.lda; }
__host__ __device__ inline const float *b_col_start(const Problem &p, std::int64_t c) { return p.tb ? p.B + c * p.ldb : p.B + c; }

// The reduced-precision workload: A and B hold 16-bit encodings (bf16 or
// f16), products are summed in FP32, C is FP32; otherwise as Problem.
enum class LpType { BF16, F16 };
struct LpProblem {
    const std::uint16_t *A;
    const std::uint16_t *B;
    float *C;
    std::int64_t lda, ldb, ldc;
    int M, N, K;
    int cus;
    bool ta, tb;
    float alpha, beta;
};
hipError_t launch_lowp_bf16(const LpProblem &p, hipStream_t stream);
hipError_t launch_lowp_f16(const LpProblem &p, hipStream_t stream);

// Devices the per-device caches cover (device ordinals 0 .. kMaxDevices-1).
constexpr int kMaxDevices = 64;
// Compute units of the calling thread's current device if it is a gfx950,
// else 0 (also for an ordinal past kMaxDevices). Cached per device.
int current_gfx950_cus();

// Largest grid extent used along y (row blocks); kernels loop over the rest.
constexpr unsigned kMaxGridY = 65535;

// Splits a product over a 1-D grid of BM x BN tiles into bands of at most
// max_tiles tiles each (2^22 by default, far inside the grid limit; work-group
// size times max_tiles must stay under 2^32 work-items) and calls
// launch(sub, tiles_m, tiles_n) for each band. A band is itself a product:
// op(A) and C start at its first row, op(B) and C at its first column. Band
// edges fall on multiples of BM and BN, so 16-byte alignment of the operands
// carries over.
template <int BM, int BN, class Launch>
hipError_t for_each_band(const Problem &p, Launch &&launch, std::int64_t max_tiles = std::int64_t(1) << 22)
{
    const std::int64_t kMaxTiles = max_tiles;
    const std::int64_t tiles_n_all = (std::int64_t(p.N) + BN - 1) / BN;
    const std::int64_t band_tn = tiles_n_all < kMaxTiles ? tiles_n_all : kMaxTiles;
    const std::int64_t band_tm = kMaxTiles / band_tn;
    for (std::int64_t r0 = 0; r0 < p.M; r0 += band_tm * BM) {
        for (std::int64_t c0 = 0; c0 < p.N; c0 += band_tn * BN) {
            Problem q = p;
            q.M = int(p.M - r0 < band_tm * BM ? p.M - r0 : band_tm * BM);
            q.N = int(p.N - c0 < band_tn * BN ? p.N - c0 : band_tn * BN);
            q.A = a_row_start(p, r0);
            q.B = b_col_start(p, c0);
            q.C = p.C + r0 * p.ldc + c0;
            const int tiles_m = int((q.M + BM - 1) / BM), tiles_n = int((q.N + BN - 1) / BN);
            const hipError_t e = launch(q, tiles_m, tiles_n);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

inline bool aligned16(const void *ptr) { return (reinterpret_cast<std::uintptr_t>(ptr) & 15u) == 0; }

// True when every row of A, B and C starts on a 16-byte boundary, so 4-wide
// chunks at column offsets that are multiples of 4 can move as one 128-bit
// access.
inline bool rows_aligned16(const Problem &p)
{
    return aligned16(p.A) && aligned16(p.B) && aligned16(p.C) && p.lda % 4 == 0 && p.ldb % 4 == 0 &&
           p.ldc % 4 == 0;
}

}  // namespace sgemm_impl

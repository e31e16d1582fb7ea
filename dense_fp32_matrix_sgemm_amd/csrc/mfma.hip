// Rung 4: the LDS-tiled, double-buffered product fed to the CDNA matrix cores
// with v_mfma_f32_32x32x2_f32 (FP32 operands, FP32 accumulation). The pages'
// kernels stop at register blocking on CUDA cores ("Matrix Multiplication --
// Naive to Tiled", section 07, which names tensor-core MMA only for FP16
// inputs); on gfx950 the FP32 dense contraction itself has a matrix-core
// instruction, and it is what the tile hierarchy below feeds.
//
// Hierarchy
//  * work-group: BM x BN tile of C, WAVES_M x WAVES_N waves, K walked in
//    slabs of BK; slab t+1 is fetched into registers while slab t is
//    multiplied out of LDS, then written to the other of two LDS buffers
//    (one barrier per slab);
//  * wave: WM x WN = (BM / WAVES_M) x (BN / WAVES_N) tile, held as
//    MI x (NJ * TI) accumulator blocks of 32 x 32 (16 VGPRs each);
//  * instruction: v_mfma_f32_32x32x2_f32, C[32x32] += A[32x2] * B[2x32].
//    Lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32]; accumulator
//    register r of lane l is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
//
// Operand order. The K order inside a slab is free (any order of the terms
// gives the sum), so it is chosen to make every LDS read wide:
//  * within a group of 8 consecutive k, MFMA step s (0..3) gives lane half h
//    the k index 4h + s. A lane then needs A[i][4h .. 4h+3] for the four steps:
//    one 16-byte read from the row-major A tile;
//  * the 32 columns of one MFMA block are interleaved TI-ways: block t of a
//    column group covers columns TI*c + t, c = 0..31. Lane c then reads the TI
//    adjacent values B[k][TI*c .. TI*c+TI-1] of the row-major B tile in one
//    read and feeds element t to block t. In the epilogue the same lane holds
//    TI adjacent columns of C and stores them with one wide store.
// A rows in LDS carry 4 words of padding so the 32 rows read by a half-wave at
// the same k fall in distinct banks; B rows are read as contiguous spans and
// are not padded.
//
// Ragged shapes: tiles and slabs that cross the edge of A, B or C load zeros
// outside and drop stores outside; interior tiles take the unguarded path.
#include "gemm.hpp"
#include "tile_io.hpp"

namespace sgemm_impl {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

template <int N>
struct Vec;
template <>
struct Vec<1> {
    using T = float;
};
template <>
struct Vec<2> {
    using T = float2;
};
template <>
struct Vec<4> {
    using T = float4;
};

[[maybe_unused]] __device__ __forceinline__ float elem(float v, int) { return v; }
__device__ __forceinline__ float elem(float2 v, int t) { return t == 0 ? v.x : v.y; }
__device__ __forceinline__ float elem(float4 v, int t) { return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w; }

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct MfmaConfig {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int MI = WM / 32;
    static constexpr int TI = WN >= 128 ? 4 : WN / 32;
    static constexpr int NJ = WN / (32 * TI);
    static constexpr int kPadA = 4;
    static constexpr int kPitchA = BK + kPadA;
    static constexpr int kChunksA = BM * BK / 4 / kThreads;  // 4-wide chunks per work-item
    static constexpr int kChunksB = BK * BN / 4 / kThreads;
    static constexpr int kGroupM = 8;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(TI == 1 || TI == 2 || TI == 4, "column interleave must be 1, 2 or 4");
    static_assert(WN == 32 * TI * NJ, "wave tile width must split into interleaved groups");
    static_assert(BK % 8 == 0, "slab depth must be whole groups of 8");
    static_assert(kChunksA * 4 * kThreads == BM * BK && kChunksB * 4 * kThreads == BK * BN,
                  "tiles must split evenly over the work-items");
    static constexpr std::size_t kLdsBytes = sizeof(float) * 2 * (BM * kPitchA + BK * BN);
};

template <class Cfg, bool VEC>
__global__ __launch_bounds__(Cfg::kThreads) void mfma_kernel(Problem p, int tiles_m)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
    constexpr int MI = Cfg::MI, NJ = Cfg::NJ, TI = Cfg::TI;
    constexpr int PA = Cfg::kPitchA;
    using VecB = typename Vec<TI>::T;

    __shared__ __attribute__((aligned(16))) float As[2][BM * PA];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * BN];

    int tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, Cfg::kGroupM, tm, tn);
    const std::int64_t m0 = std::int64_t(tm) * BM;
    const int n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int l32 = lane % 32, h = lane / 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wm0 = (wave / Cfg::WAVES_N) * Cfg::WM;
    const int wn0 = (wave % Cfg::WAVES_N) * Cfg::WN;

    const bool rows_in = m0 + BM <= p.M;
    const bool cols_in = n0 + BN <= p.N;
    const int n_slabs = (p.K + BK - 1) / BK;

    floatx16 acc[MI][NJ][TI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int t = 0; t < TI; ++t) acc[mi][nj][t] = floatx16{};

    float4 ra[Cfg::kChunksA], rb[Cfg::kChunksB];

    auto fetch = [&](int slab) {
        const int k0 = slab * BK;
        const bool k_in = k0 + BK <= p.K;
#pragma unroll
        for (int q = 0; q < Cfg::kChunksA; ++q) {
            const int c = tid + q * Cfg::kThreads;
            const int row = c / (BK / 4), kk = (c % (BK / 4)) * 4;
            ra[q] = load4<VEC>(p.A, p.lda, m0 + row, k0 + kk, p.M, p.K, rows_in && k_in);
        }
#pragma unroll
        for (int q = 0; q < Cfg::kChunksB; ++q) {
            const int c = tid + q * Cfg::kThreads;
            const int kr = c / (BN / 4), col = (c % (BN / 4)) * 4;
            rb[q] = load4<VEC>(p.B, p.ldb, k0 + kr, n0 + col, p.K, p.N, k_in && cols_in);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int q = 0; q < Cfg::kChunksA; ++q) {
            const int c = tid + q * Cfg::kThreads;
            const int row = c / (BK / 4), kk = (c % (BK / 4)) * 4;
            *reinterpret_cast<float4 *>(&As[buf][row * PA + kk]) = ra[q];
        }
#pragma unroll
        for (int q = 0; q < Cfg::kChunksB; ++q) {
            const int c = tid + q * Cfg::kThreads;
            const int kr = c / (BN / 4), col = (c % (BN / 4)) * 4;
            *reinterpret_cast<float4 *>(&Bs[buf][kr * BN + col]) = rb[q];
        }
    };
    auto multiply = [&](int buf) {
        const float *as = As[buf];
        const float *bs = Bs[buf];
#pragma unroll
        for (int g = 0; g < BK / 8; ++g) {
            float4 af[MI];
            VecB bf[4][NJ];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                af[mi] = *reinterpret_cast<const float4 *>(&as[(wm0 + mi * 32 + l32) * PA + 8 * g + 4 * h]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int nj = 0; nj < NJ; ++nj)
                    bf[s][nj] = *reinterpret_cast<const VecB *>(
                        &bs[(8 * g + 4 * h + s) * BN + wn0 + nj * 32 * TI + l32 * TI]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
                        for (int t = 0; t < TI; ++t)
                            acc[mi][nj][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                elem(af[mi], s), elem(bf[s][nj], t), acc[mi][nj][t], 0, 0, 0);
        }
    };

    if (n_slabs > 0) {
        fetch(0);
        stash(0);
        __syncthreads();
        for (int t = 0; t < n_slabs; ++t) {
            const int cur = t & 1;
            const bool more = t + 1 < n_slabs;
            if (more) fetch(t + 1);
            multiply(cur);
            if (more) stash(cur ^ 1);
            __syncthreads();
        }
    }

    // Epilogue: register r of block (mi, nj, t) is row 8(r/4) + 4h + r%4 of
    // the block and column TI*l32 + t of the column group.
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const std::int64_t row = m0 + wm0 + mi * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                const int col = n0 + wn0 + nj * 32 * TI + l32 * TI;
                float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t = 0; t < TI; ++t) v[t] = acc[mi][nj][t][r];
                if constexpr (TI == 4) {
                    store4<VEC>(p.C, p.ldc, row, col, p.M, p.N, make_float4(v[0], v[1], v[2], v[3]));
                } else {
                    if (row < p.M) {
#pragma unroll
                        for (int t = 0; t < TI; ++t)
                            if (col + t < p.N) p.C[row * p.ldc + col + t] = v[t];
                    }
                }
            }
}

using DefaultCfg = MfmaConfig<128, 128, 16, 2, 2>;

template <class Cfg>
hipError_t launch_cfg(const Problem &p, hipStream_t stream)
{
    const void *kernel = rows_aligned16(p) ? reinterpret_cast<const void *>(&mfma_kernel<Cfg, true>)
                                           : reinterpret_cast<const void *>(&mfma_kernel<Cfg, false>);
    return for_each_band<Cfg::BM, Cfg::BN>(p, [&](Problem q, int tiles_m, int tiles_n) {
        void *args[] = {&q, &tiles_m};
        return hipLaunchKernel(kernel, dim3(unsigned(tiles_m) * unsigned(tiles_n)), dim3(Cfg::kThreads), args, 0,
                               stream);
    });
}

}  // namespace

hipError_t launch_mfma(const Problem &p, hipStream_t stream) { return launch_cfg<DefaultCfg>(p, stream); }

}  // namespace sgemm_impl

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
#include <type_traits>

#include "gemm.hpp"
#include "tile_io.hpp"

namespace sgemm_impl {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
// Native 4-wide vector: copies of it stay in registers (copies of the HIP
// float4 struct through pointers become memcpy and can end up in scratch).
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
    static constexpr int kLdsFloats = 2 * (BM * kPitchA + BK * BN);  // two stages of A and B tiles
    static constexpr int kChunksA = BM * BK / 4 / kThreads;  // 4-wide chunks per work-item
    static constexpr int kChunksB = BK * BN / 4 / kThreads;
#ifndef SGEMM_MFMA_GROUP_M
#define SGEMM_MFMA_GROUP_M 8
#endif
    static constexpr int kGroupM = SGEMM_MFMA_GROUP_M;
    // Waves per SIMD the register allocation aims at: one when a wave's
    // accumulators alone fill the 256 AGPRs, more as they shrink.
    static constexpr int kWavesPerEU = MI * NJ * TI * 16 >= 256 ? 1 : MI * NJ * TI * 16 >= 64 ? 2 : 4;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(TI == 1 || TI == 2 || TI == 4, "column interleave must be 1, 2 or 4");
    static_assert(WN == 32 * TI * NJ, "wave tile width must split into interleaved groups");
    static_assert(BK % 8 == 0, "slab depth must be whole groups of 8");
    static_assert(kChunksA * 4 * kThreads == BM * BK && kChunksB * 4 * kThreads == BK * BN,
                  "tiles must split evenly over the work-items");
    static constexpr std::size_t kLdsBytes = sizeof(float) * 2 * (BM * kPitchA + BK * BN);
};

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100, kSchedDsWrite = 0x200;

// One BM x BN tile (tm, tn) of the product p, with guards on every edge;
// `lds` holds Cfg::kLdsFloats floats.
template <class Cfg, bool VEC>
__device__ __forceinline__ void general_tile(const Problem &p, int tm, int tn, float *lds)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
    constexpr int MI = Cfg::MI, NJ = Cfg::NJ, TI = Cfg::TI;
    constexpr int PA = Cfg::kPitchA;
    constexpr int G = BK / 8;  // groups of 8 k per slab
    using VecB = typename Vec<TI>::T;

    float(*As)[BM * PA] = reinterpret_cast<float(*)[BM * PA]>(lds);
    float(*Bs)[BK * BN] = reinterpret_cast<float(*)[BK * BN]>(lds + 2 * BM * PA);

    const std::int64_t m0 = std::int64_t(tm) * BM;
    const int n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int l32 = lane % 32, h = lane / 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wm0 = (wave / Cfg::WAVES_N) * Cfg::WM;
    const int wn0 = (wave % Cfg::WAVES_N) * Cfg::WN;

    // Interior tiles run the pipelined loop over their whole slabs with
    // unguarded loads and finish a partial last slab separately; edge tiles
    // run the same loop with guarded loads throughout. The two loops are
    // separate instantiations, so the guarded path's addresses are never
    // live in the fast one.
    const bool interior = m0 + BM <= p.M && n0 + BN <= p.N;
    const int n_slabs = (p.K + BK - 1) / BK;
    const int n_full = p.K / BK;

    floatx16 acc[MI][NJ][TI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int t = 0; t < TI; ++t) acc[mi][nj][t] = floatx16{};

    // Global -> register staging of one slab: chunk c of the A tile is row
    // c / (BK/4), columns 4 (c % (BK/4)) ..; chunk c of the B tile is row
    // c / (BN/4), columns 4 (c % (BN/4)) ...
    float4 ra[Cfg::kChunksA], rb[Cfg::kChunksB];
    auto fetch = [&](int slab, auto guarded) {
        const int k0 = slab * BK;
#pragma unroll
        for (int q = 0; q < Cfg::kChunksA; ++q) {
            const int c = tid + q * Cfg::kThreads;
            const std::int64_t row = m0 + c / (BK / 4);
            const int col = k0 + (c % (BK / 4)) * 4;
            if constexpr (decltype(guarded)::value)
                ra[q] = load4_clamped(p.A, p.lda, row, col, p.M, p.K);
            else
                ra[q] = load4_inside<VEC>(p.A, p.lda, row, col);
        }
#pragma unroll
        for (int q = 0; q < Cfg::kChunksB; ++q) {
            const int c = tid + q * Cfg::kThreads;
            const std::int64_t row = k0 + c / (BN / 4);
            const int col = n0 + (c % (BN / 4)) * 4;
            if constexpr (decltype(guarded)::value)
                rb[q] = load4_clamped(p.B, p.ldb, row, col, p.K, p.N);
            else
                rb[q] = load4_inside<VEC>(p.B, p.ldb, row, col);
        }
    };
    auto stash = [&](int buf, int slab, auto guarded) {
        if constexpr (decltype(guarded)::value) {
            const int k0 = slab * BK;
#pragma unroll
            for (int q = 0; q < Cfg::kChunksA; ++q) {
                const int c = tid + q * Cfg::kThreads;
                zero_outside(ra[q], m0 + c / (BK / 4), k0 + (c % (BK / 4)) * 4, p.M, p.K);
            }
#pragma unroll
            for (int q = 0; q < Cfg::kChunksB; ++q) {
                const int c = tid + q * Cfg::kThreads;
                zero_outside(rb[q], k0 + c / (BN / 4), n0 + (c % (BN / 4)) * 4, p.K, p.N);
            }
        }
#pragma unroll
        for (int q = 0; q < Cfg::kChunksA; ++q) {
            const int c = tid + q * Cfg::kThreads;
            *reinterpret_cast<float4 *>(&As[buf][(c / (BK / 4)) * PA + (c % (BK / 4)) * 4]) = ra[q];
        }
#pragma unroll
        for (int q = 0; q < Cfg::kChunksB; ++q) {
            const int c = tid + q * Cfg::kThreads;
            *reinterpret_cast<float4 *>(&Bs[buf][(c / (BN / 4)) * BN + (c % (BN / 4)) * 4]) = rb[q];
        }
    };

    // Operand fragments of one group of 8 k, double-buffered in registers so
    // the reads of group g+1 are in flight while group g's MFMAs issue.
    float4 af[2][MI];
    VecB bf[2][4][NJ];
    auto read_frags = [&](int buf, int g, int slot) {
        const float *as = As[buf];
        const float *bs = Bs[buf];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            af[slot][mi] = *reinterpret_cast<const float4 *>(&as[(wm0 + mi * 32 + l32) * PA + 8 * g + 4 * h]);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj)
                bf[slot][s][nj] =
                    *reinterpret_cast<const VecB *>(&bs[(8 * g + 4 * h + s) * BN + wn0 + nj * 32 * TI + l32 * TI]);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
                    for (int t = 0; t < TI; ++t)
                        acc[mi][nj][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            elem(af[slot][mi], s), elem(bf[slot][s][nj], t), acc[mi][nj][t], 0, 0, 0);
    };
    // Multiply out one LDS buffer; `between` runs half-way through.
    auto multiply = [&](int buf, auto &&between) {
        read_frags(buf, 0, 0);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g + 1 < G) read_frags(buf, g + 1, (g + 1) & 1);
            if (g == G / 2) between();
            mfmas(g & 1);
        }
    };

    // Slabs [0, n) with the two-buffer pipeline: slab t+1 waits in registers
    // while slab t is multiplied; half-way through slab t it is written to the
    // other LDS buffer (which every wave finished reading before the previous
    // barrier) and the fetch of slab t+2 starts.
    auto pipeline = [&](int n, auto guarded) {
        if (n <= 0) return;
        fetch(0, guarded);
        stash(0, 0, guarded);
        if (n > 1) fetch(1, guarded);
        __syncthreads();
        for (int t = 0; t < n; ++t) {
            const int cur = t & 1;
            multiply(cur, [&] {
                if (t + 1 < n) {
                    stash(cur ^ 1, t + 1, guarded);
                    if (t + 2 < n) fetch(t + 2, guarded);
                }
            });
            __syncthreads();
        }
    };

    if (interior) {
        pipeline(n_full, std::false_type{});
        if (n_full < n_slabs) {  // partial last slab
            fetch(n_full, std::true_type{});
            stash(0, n_full, std::true_type{});
            __syncthreads();
            multiply(0, [] {});
        }
    } else {
        pipeline(n_slabs, std::true_type{});
    }

    // Epilogue: register r of block (mi, nj, t) is row 8(r/4) + 4h + r%4 of
    // the block and column TI*l32 + t of its column group.
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const std::int64_t row = m0 + wm0 + mi * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                const int col = n0 + wn0 + nj * 32 * TI + l32 * TI;
                float v[TI];
#pragma unroll
                for (int t = 0; t < TI; ++t) v[t] = acc[mi][nj][t][r];
                store_n<VEC, TI>(p.C, p.ldc, row, col, p.M, p.N, v, interior);
            }
}

// Interior tiles: the tile lies wholly inside C and the slab loop carries
// no guard at all. Rows need only the 4-byte alignment of any float: global
// memory moves in 16-byte accesses that gfx950 performs unaligned. The partial
// last slab (K not a multiple of BK) is loaded once, with guards, after the
// loop. Same operand order and LDS layout as general_tile; the slab loop is
// arranged for a single wave per SIMD:
//  * each steady-state slab is one straight-line block whose LDS stores,
//    global loads and fragment reads are spread one per MFMA (a burst of
//    memory instructions would hold back the next MFMA, as a wave issues in
//    order);
//  * the barrier sits before the last group of k of the slab, so the first
//    fragments of the next slab load while that group is multiplied.
// interior_tile computes one whole BM x BN tile (tm, tn) of the product p
// (no edge inside it); `lds` holds Cfg::kLdsFloats floats.
template <class Cfg>
__device__ __forceinline__ void interior_tile(const Problem &p, int tm, int tn, float *lds)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::kThreads;
    constexpr int MI = Cfg::MI, NJ = Cfg::NJ, TI = Cfg::TI;
    constexpr int PA = Cfg::kPitchA;
    constexpr int G = BK / 8;
    constexpr int CA = Cfg::kChunksA, CB = Cfg::kChunksB;
    using VecB = typename Vec<TI>::T;

    float(*As)[BM * PA] = reinterpret_cast<float(*)[BM * PA]>(lds);
    float(*Bs)[BK * BN] = reinterpret_cast<float(*)[BK * BN]>(lds + 2 * BM * PA);

    const std::int64_t m0 = std::int64_t(tm) * BM;
    const int n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int l32 = lane % 32, h = lane / 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wm0 = (wave / Cfg::WAVES_N) * Cfg::WM;
    const int wn0 = (wave % Cfg::WAVES_N) * Cfg::WN;
    const int n_full = p.K / BK;

    floatx16 acc[MI][NJ][TI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int t = 0; t < TI; ++t) acc[mi][nj][t] = floatx16{};

    // This work-item's chunks: A chunk q is row (q*NT + tid) / (BK/4) of the
    // tile, columns 4 ((q*NT + tid) % (BK/4)) ..; B chunk q is row
    // (q*NT + tid) / (BN/4), columns 4 ((q*NT + tid) % (BN/4)) ...
    const float *ga = p.A + (m0 + tid / (BK / 4)) * p.lda + (tid % (BK / 4)) * 4;
    const float *gb = p.B + std::int64_t(tid / (BN / 4)) * p.ldb + n0 + (tid % (BN / 4)) * 4;
    constexpr int kRowStepA = NT / (BK / 4);  // tile rows between consecutive chunks q
    constexpr int kRowStepB = NT / (BN / 4);
    static_assert(NT % (BK / 4) == 0 && NT % (BN / 4) == 0, "chunk rows must advance evenly");

    f32x4 ra[CA], rb[CB];
    auto fetch = [&](int slab) {
        const std::int64_t ka = std::int64_t(slab) * BK, kb = std::int64_t(slab) * BK * p.ldb;
#pragma unroll
        for (int q = 0; q < CA; ++q)
            ra[q] = load16u(ga + q * kRowStepA * p.lda + ka);
#pragma unroll
        for (int q = 0; q < CB; ++q)
            rb[q] = load16u(gb + q * kRowStepB * p.ldb + kb);
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int q = 0; q < CA; ++q) {
            const int c = q * NT + tid;
            *reinterpret_cast<f32x4 *>(&As[buf][(c / (BK / 4)) * PA + (c % (BK / 4)) * 4]) = ra[q];
        }
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            const int c = q * NT + tid;
            *reinterpret_cast<f32x4 *>(&Bs[buf][(c / (BN / 4)) * BN + (c % (BN / 4)) * 4]) = rb[q];
        }
    };

    float4 af[2][MI];
    VecB bf[2][4][NJ];
    auto read_frags = [&](int buf, int g, int slot) {
        const float *as = As[buf];
        const float *bs = Bs[buf];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            af[slot][mi] = *reinterpret_cast<const float4 *>(&as[(wm0 + mi * 32 + l32) * PA + 8 * g + 4 * h]);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj)
                bf[slot][s][nj] =
                    *reinterpret_cast<const VecB *>(&bs[(8 * g + 4 * h + s) * BN + wn0 + nj * 32 * TI + l32 * TI]);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
                    for (int t = 0; t < TI; ++t)
                        acc[mi][nj][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            elem(af[slot][mi], s), elem(bf[slot][s][nj], t), acc[mi][nj][t], 0, 0, 0);
    };
    auto multiply = [&](int buf, auto &&between) {
        read_frags(buf, 0, 0);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g + 1 < G) read_frags(buf, g + 1, (g + 1) & 1);
            if (g == G / 2) between();
            mfmas(g & 1);
        }
    };

    static_assert(G % 2 == 0, "the pipelined loop needs an even number of k-groups per slab");
    constexpr int NR = MI + 4 * NJ;            // fragment reads per group
    // Interleave hints: one memory instruction after each MFMA, so no burst
    // of loads or stores holds back the next MFMA in the wave's in-order issue.
    auto interleave_a = [&] {
#pragma unroll
        for (int i = 0; i < (G - 1) * NR; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < CA + CB; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < CA + CB; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
        }
    };
    auto interleave_b = [&] {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
    };

    const int n = n_full;
    if (n > 0) {
        fetch(0);
        stash(0);
        if (n > 1) fetch(1);
        __syncthreads();
        read_frags(0, 0, 0);
        int t = 0;
        // Steady state, one straight-line block per slab t (LDS buffer cur):
        //   A: store slab t+1 (registers) to buffer cur^1, start loading slab
        //      t+2, read groups 1..G-1 of slab t while multiplying groups
        //      0..G-2;
        //   barrier: slab t+1 is complete in LDS, and every wave has finished
        //      reading buffer cur^1's previous contents (slab t-1, before the
        //      previous barrier);
        //   B: read group 0 of slab t+1 while multiplying group G-1 of slab t.
        for (; t + 2 < n; ++t) {
            const int cur = t & 1;
            stash(cur ^ 1);
            fetch(t + 2);
#pragma unroll
            for (int g = 0; g + 1 < G; ++g) {
                read_frags(cur, g + 1, (g + 1) & 1);
                mfmas(g & 1);
            }
            interleave_a();
            __syncthreads();
            read_frags(cur ^ 1, 0, 0);
            mfmas((G - 1) & 1);
            interleave_b();
        }
        // Last two slabs: no more loads.
        for (; t < n; ++t) {
            const int cur = t & 1;
            if (t + 1 < n) stash(cur ^ 1);
#pragma unroll
            for (int g = 0; g + 1 < G; ++g) {
                read_frags(cur, g + 1, (g + 1) & 1);
                mfmas(g & 1);
            }
            __syncthreads();
            if (t + 1 < n) read_frags(cur ^ 1, 0, 0);
            mfmas((G - 1) & 1);
        }
        __syncthreads();
    }
    if (n_full * BK < p.K) {
        // Partial last slab: columns k >= K of A and rows k >= K of B read as
        // zero. Written straight to LDS one element at a time; this runs once.
        const int k0 = n_full * BK;
#pragma unroll 1
        for (int e = tid; e < BM * BK; e += NT) {
            const int r = e / BK, k = e % BK;
            As[0][r * PA + k] = k0 + k < p.K ? p.A[(m0 + r) * p.lda + k0 + k] : 0.0f;
        }
#pragma unroll 1
        for (int e = tid; e < BK * BN; e += NT) {
            const int k = e / BN, c = e % BN;
            Bs[0][k * BN + c] = k0 + k < p.K ? p.B[std::int64_t(k0 + k) * p.ldb + n0 + c] : 0.0f;
        }
        __syncthreads();
        multiply(0, [] {});
    }

#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const std::int64_t row = m0 + wm0 + mi * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                const int col = n0 + wn0 + nj * 32 * TI + l32 * TI;
                float *c = p.C + row * p.ldc + col;
                if constexpr (TI == 4) {
                    store16u(c, f32x4{acc[mi][nj][0][r], acc[mi][nj][1][r], acc[mi][nj][2][r], acc[mi][nj][3][r]});
                } else if constexpr (TI == 2) {
                    store8u(c, acc[mi][nj][0][r], acc[mi][nj][1][r]);
                } else {
                    c[0] = acc[mi][nj][0][r];
                }
            }
}

#ifndef SGEMM_MFMA_TILE
#define SGEMM_MFMA_TILE 128, 128, 32, 2, 2
#endif
#ifndef SGEMM_MFMA_BIG_TILE
#define SGEMM_MFMA_BIG_TILE 256, 256, 16, 2, 2
#endif
#ifndef SGEMM_MFMA_MID_TILE
#define SGEMM_MFMA_MID_TILE 128, 128, 32, 2, 2
#endif
#ifndef SGEMM_MFMA_SMALL_TILE
#define SGEMM_MFMA_SMALL_TILE 64, 64, 32, 2, 2
#endif
// Tile shapes (BM, BN, BK, WAVES_M, WAVES_N): the general tiles (edges) and
// three sizes of interior tile.
using GeneralCfg = MfmaConfig<SGEMM_MFMA_TILE>;
using BigCfg = MfmaConfig<SGEMM_MFMA_BIG_TILE>;
using MidCfg = MfmaConfig<SGEMM_MFMA_MID_TILE>;
using SmallCfg = MfmaConfig<SGEMM_MFMA_SMALL_TILE>;

template <class A, class B>
constexpr int max_lds() { return A::kLdsFloats > B::kLdsFloats ? A::kLdsFloats : B::kLdsFloats; }

// Products too small for a single interior tile: general tiles only.
template <class Cfg, bool VEC>
__global__ __launch_bounds__(Cfg::kThreads) void mfma_kernel(Problem p, int tiles_m)
{
    __shared__ __attribute__((aligned(16))) float lds[Cfg::kLdsFloats];
    int tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, Cfg::kGroupM, tm, tn);
    general_tile<Cfg, VEC>(p, tm, tn, lds);
}

// Work-group layout of one fused launch: first the interior tiles (whole
// ICfg tiles covering rows [0, mi) and columns [0, ni)), then the general
// tiles of the bottom strip (rows [mi, M), all columns) and of the right
// strip (rows [0, mi), columns [ni, N)).
struct FusedGrid {
    unsigned n_interior, n_bottom;
    int tiles_m;              // interior tile rows
    int bottom_tn, right_tn;  // general tiles per row of each strip
    int mi, ni;
};

// One launch for the whole product, so the small strips run beside the
// interior tiles instead of after them; the two bodies share one LDS buffer.
template <class A, class B>
constexpr int min_waves() { return A::kWavesPerEU < B::kWavesPerEU ? A::kWavesPerEU : B::kWavesPerEU; }

template <class ICfg, class GCfg, bool VEC>
__global__ __launch_bounds__(ICfg::kThreads)
__attribute__((amdgpu_waves_per_eu(min_waves<ICfg, GCfg>(), min_waves<ICfg, GCfg>()))) void mfma_fused_kernel(
    Problem p, FusedGrid g)
{
    static_assert(ICfg::kThreads == GCfg::kThreads, "both bodies run in the same work-group shape");
    __shared__ __attribute__((aligned(16))) float lds[max_lds<ICfg, GCfg>()];
    const unsigned w = blockIdx.x;
    if (w < g.n_interior) {
        int tm, tn;
        tile_of_workgroup(w, g.n_interior, g.tiles_m, ICfg::kGroupM, tm, tn);
        interior_tile<ICfg>(p, tm, tn, lds);
        return;
    }
    unsigned e = w - g.n_interior;
    Problem q = p;
    int tm, tn;
    if (e < g.n_bottom) {
        q.M = p.M - g.mi;
        if (p.K > 0) q.A = p.A + std::int64_t(g.mi) * p.lda;
        q.C = p.C + std::int64_t(g.mi) * p.ldc;
        tm = int(e / unsigned(g.bottom_tn));
        tn = int(e % unsigned(g.bottom_tn));
    } else {
        e -= g.n_bottom;
        q.M = g.mi;
        q.N = p.N - g.ni;
        if (p.K > 0) q.B = p.B + g.ni;
        q.C = p.C + g.ni;
        tm = int(e / unsigned(g.right_tn));
        tn = int(e % unsigned(g.right_tn));
    }
    general_tile<GCfg, VEC>(q, tm, tn, lds);
}

template <class Cfg>
hipError_t launch_general(const Problem &p, hipStream_t stream)
{
    const void *kernel = rows_aligned16(p) ? reinterpret_cast<const void *>(&mfma_kernel<Cfg, true>)
                                           : reinterpret_cast<const void *>(&mfma_kernel<Cfg, false>);
    return for_each_band<Cfg::BM, Cfg::BN>(p, [&](Problem q, int tiles_m, int tiles_n) {
        void *args[] = {&q, &tiles_m};
        return hipLaunchKernel(kernel, dim3(unsigned(tiles_m) * unsigned(tiles_n)), dim3(Cfg::kThreads), args, 0,
                               stream);
    });
}

template <class Cfg>
std::int64_t whole_tiles(const Problem &p)
{
    return std::int64_t(p.M / Cfg::BM) * std::int64_t(p.N / Cfg::BN);
}

template <class ICfg, class GCfg>
hipError_t launch_fused(const Problem &p, hipStream_t stream)
{
    return for_each_band<ICfg::BM, ICfg::BN>(p, [&](Problem q, int, int) {
        const int mi = q.M / ICfg::BM * ICfg::BM, ni = q.N / ICfg::BN * ICfg::BN;
        if (mi == 0 || ni == 0) return launch_general<GeneralCfg>(q, stream);
        FusedGrid g;
        g.tiles_m = mi / ICfg::BM;
        g.n_interior = unsigned(g.tiles_m) * unsigned(ni / ICfg::BN);
        g.mi = mi;
        g.ni = ni;
        g.bottom_tn = (q.N + GCfg::BN - 1) / GCfg::BN;
        g.right_tn = (q.N - ni + GCfg::BN - 1) / GCfg::BN;
        g.n_bottom = mi < q.M ? unsigned((q.M - mi + GCfg::BM - 1) / GCfg::BM) * unsigned(g.bottom_tn) : 0u;
        const unsigned n_right = ni < q.N ? unsigned((mi + GCfg::BM - 1) / GCfg::BM) * unsigned(g.right_tn) : 0u;
        const void *kernel = rows_aligned16(q) ? reinterpret_cast<const void *>(&mfma_fused_kernel<ICfg, GCfg, true>)
                                               : reinterpret_cast<const void *>(&mfma_fused_kernel<ICfg, GCfg, false>);
        void *args[] = {&q, &g};
        return hipLaunchKernel(kernel, dim3(g.n_interior + g.n_bottom + n_right), dim3(ICfg::kThreads), args, 0,
                               stream);
    });
}

// Tile size by shape: the largest interior tile whose whole tiles alone
// give every compute unit at least one work-group (one 256x256 tile per CU
// already keeps all four SIMDs of the CU busy); smaller products fall back
// to 128x128 and then 64x64 tiles, which trade operand reuse for parallelism.
// The strips of a 256x256 split use 128x128 general tiles; the smaller
// splits use general tiles of their own size.
hipError_t launch_by_shape(const Problem &p, hipStream_t stream)
{
    const std::int64_t fill = p.cus > 0 ? p.cus : 256;
    if (whole_tiles<BigCfg>(p) >= fill) return launch_fused<BigCfg, GeneralCfg>(p, stream);
    if (whole_tiles<MidCfg>(p) >= fill) return launch_fused<MidCfg, MidCfg>(p, stream);
    return launch_fused<SmallCfg, SmallCfg>(p, stream);
}

}  // namespace

hipError_t launch_mfma(const Problem &p, hipStream_t stream) { return launch_by_shape(p, stream); }

}  // namespace sgemm_impl

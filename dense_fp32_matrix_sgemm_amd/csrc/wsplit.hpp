// Matrix-core tiles for products that give each compute unit about one tile
// of C (1024^3 has 256 tiles of 64 x 64 for 256 compute units, 1536^3 256 of
// 96 x 96, 2048^3 256 of 128 x 128): the work-group's four waves each compute
// the WHOLE tile over a quarter of K, and the four partial tiles are summed
// at the end. Splitting K this way is free: the terms of a dot product may
// be added in any grouping ("Matrix Multiplication -- Naive to Tiled",
// section 07 on split-K), and here the grouping is fixed, so every run gives
// the same bits.
//
// Why not the LDS-staged loop of the other tiles: with one tile per compute
// unit, the loop spends its time on the barrier of every slab and the wait
// for the fragments read after it. Here a wave shares nothing with the
// others until the end, so the loop has no LDS and no barrier:
//  * a wave reads its operands straight from global memory (L2) into
//    registers, already in the order v_mfma_f32_32x32x2_f32 takes them, one
//    chunk of k ahead of the one it multiplies (a chunk of a 64 x 64 tile is
//    64 MFMAs, about 1.7 us: longer than a load's round trip);
//  * buffer loads carry the per-lane part of each address in one VGPR and the
//    per-row and per-chunk parts in scalar registers, so the loop issues no
//    vector address arithmetic between its MFMAs;
//  * chunk c belongs to wave c % 4; the partial tiles meet once, in LDS (in
//    two rounds of block rows for the 128 x 128 tile, whose four partial
//    tiles would not fit at once).
//
// A tile of NB x NB blocks of 32 x 32 (NB = 2, 3, 4). K order inside a chunk
// of CH values (k0 .. k0+CH-1): MFMA step s (0 .. CH/2-1) gives lane half h
// the k index k0 + (CH/2) h + s. So
//  * an operand stored with k contiguous ("KC": A as given, B transposed)
//    gives lane (l32, h) of block b the CH/2 values X[f][k0 + (CH/2) h ..] of
//    its free index f = 32b + l32 as 16-byte loads;
//  * an operand stored with its free index contiguous ("FC": B as given, A
//    transposed) gives lane (c, h) the NB values X[k0 + (CH/2) h + s][NB c ..
//    NB c + NB - 1] with one load per step; element e feeds block e, so block e
//    covers the free indices NB c + e and a lane ends up with NB adjacent
//    columns of C (B as given).
//
// Ragged shapes: a KC row past the operand's edge is read from the last row
// (its values only reach rows of C that are never stored); an FC group that
// crosses the edge is read from the last NB elements and shifted down, so its
// valid elements land in their places. The partial last chunk of K (rem = K
// mod CH values) is read element by element with zeros past K, in a k order
// of its own, k0 + 2s + h for step s and lane half h, so that its values fill
// the first ceil(rem / 2) steps and the rest are skipped. Its loads are not
// prefetched, so a ragged K costs each tile a load's round trip; the host
// takes these tiles for a ragged K only where a compute unit holds a single
// tile. This needs the FC operand at least NB wide (products under 4 wide
// take the general tiles).
#pragma once

#include <cstdint>
#include <type_traits>

#include "gemm.hpp"
#include "tile_io.hpp"

namespace sgemm_impl {
namespace {

typedef float ws_f32x16 __attribute__((ext_vector_type(16)));
typedef float ws_f32x4 __attribute__((ext_vector_type(4)));
typedef float ws_f32x3 __attribute__((ext_vector_type(3)));
typedef float ws_f32x2 __attribute__((ext_vector_type(2)));

template <int N>
struct WsVec;
template <>
struct WsVec<2> {
    using T = ws_f32x2;
};
template <>
struct WsVec<3> {
    using T = ws_f32x3;
};
template <>
struct WsVec<4> {
    using T = ws_f32x4;
};

constexpr int kWsWaves = 4;  // K split over the work-group's waves
// gfx9 buffer resource word 3 for untyped 32-bit accesses.
constexpr int kBufferWord3 = 0x00020000;

// NB x NB blocks of 32 x 32, chunks of CH k, SETS register sets a wave's
// chunks stream through (chunk i + SETS - 1 is requested while chunk i is
// multiplied), and the waves per SIMD its registers are bounded for (2 lets
// two work-groups share a compute unit).
template <int NB_, int CH_, int SETS_, int WPE_>
struct WsConfig {
    static constexpr int NB = NB_;
    static constexpr int T = 32 * NB;  // tile edge
    static constexpr int CH = CH_;
    static constexpr int S = CH / 2;  // MFMA steps per chunk
    static constexpr int SETS = SETS_;
    static constexpr int WPE = WPE_;
    // Block rows per round of the partial tiles' sum in LDS.
    static constexpr int RR = NB == 4 ? 2 : NB;
    static constexpr int kRedFloats = kWsWaves * RR * NB * 4 * 64 * 4;
    static_assert(NB >= 2 && NB <= 4, "tiles of 2 x 2 to 4 x 4 blocks");
    static_assert(CH == 16 || CH == 32, "chunks of 16 or 32 k");
    static_assert(SETS >= 2 && SETS <= 3, "two or three register sets");
    static_assert(NB % RR == 0, "whole rounds of block rows");
    static_assert(kRedFloats * 4 <= 160 * 1024, "the partial tiles fit the LDS");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const float *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, 0x7fffffff, kBufferWord3);
}

template <int N>
__device__ __forceinline__ typename WsVec<N>::T ws_load(__amdgpu_buffer_rsrc_t rs, int vo, int so)
{
    using V = typename WsVec<N>::T;
    if constexpr (N == 2)
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(rs, vo, so, 0));
    else if constexpr (N == 3)
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b96(rs, vo, so, 0));
    else
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, so, 0));
}

// An operand stored with k contiguous. The resource starts at the tile's
// first free index; lane offsets are relative to it.
template <class Cfg, bool EDGE>
struct WsKC {
    static constexpr int NB = Cfg::NB, S = Cfg::S, CH = Cfg::CH;
    static constexpr int kLoads = NB * S / 4;  // per chunk
    ws_f32x4 v[NB][S / 4];  // v[b][j][e]: k = k0 + S h + 4j + e of block b
    __amdgpu_buffer_rsrc_t rs;
    int vo[NB];            // byte offset of (free index of block b, k = S h)
    const float *row[NB];  // the same rows as plain pointers (partial chunk)

    __device__ float get(int b, int s) const { return v[b][s / 4][s % 4]; }
    __device__ static int free_index(int b, int l32) { return 32 * b + l32; }

    __device__ void init(const float *X, std::int64_t ld, std::int64_t f0, std::int64_t extent, int l32, int h)
    {
        rs = ws_rsrc(X + f0 * ld);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            std::int64_t f = f0 + 32 * b + l32;
            if (EDGE && f >= extent) f = extent - 1;
            vo[b] = int(((f - f0) * ld + S * h) * 4);
            row[b] = X + f * ld;
        }
    }
    // Full chunk c (k0 = CH c).
    __device__ void load(int c)
    {
        const int so = c * CH * 4;
#pragma unroll
        for (int j = 0; j < S / 4; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b) v[b][j] = ws_load<4>(rs, vo[b] + 16 * j, so);
    }
    // The partial chunk starting at k0, in its own k order (step s, half h:
    // k = k0 + 2s + h), with zeros at k >= K.
    __device__ void load_partial(int k0, int K, int h)
    {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int k = k0 + 2 * s + h;
                const float x = row[b][k < K ? k : K - 1];
                v[b][s / 4][s % 4] = k < K ? x : 0.0f;
            }
    }
};

// An operand stored with its free index contiguous. The resource starts at
// the operand itself (free index 0), so that an edge group can be read from
// the last NB elements wherever the tile starts.
template <class Cfg, bool EDGE>
struct WsFC {
    static constexpr int NB = Cfg::NB, S = Cfg::S, CH = Cfg::CH;
    static constexpr int kLoads = S;  // per chunk
    using V = typename WsVec<NB>::T;
    V u[S];  // u[s][e]: k = k0 + S h + s, free index NB c + e
    __amdgpu_buffer_rsrc_t rs;
    int vo, ld4;
    int shift;         // the group was read `shift` elements early (edge)
    const float *col;  // the lane's group in stored row 0 (partial chunk)
    std::int64_t ld;

    // The shift is applied where a value is used, not where it is loaded: a
    // select right after the load would wait for the load there and then.
    __device__ float get(int b, int s) const
    {
        float x = u[s][b];
        if constexpr (EDGE) {
#pragma unroll
            for (int d = 1; b + d < NB; ++d) x = shift == d ? u[s][b + d] : x;
        }
        return x;
    }
    __device__ static int free_index(int b, int l32) { return NB * l32 + b; }

    __device__ void init(const float *X, std::int64_t ld_, std::int64_t f0, std::int64_t extent, int l32, int h)
    {
        ld = ld_;
        rs = ws_rsrc(X);
        std::int64_t f = f0 + NB * l32;
        shift = 0;
        if (EDGE && f + NB > extent) {
            // Valid elements f .. extent - 1 (if any) sit at positions shift ..
            // NB - 1 of the group read from extent - NB.
            shift = f < extent ? int(f - (extent - NB)) : 0;
            f = extent - NB;
        }
        vo = int((S * h * ld + f) * 4);
        ld4 = int(ld * 4);
        col = X + f;
    }
    __device__ void load(int c)
    {
        const int so = c * CH * ld4;
#pragma unroll
        for (int s = 0; s < S; ++s) u[s] = ws_load<NB>(rs, vo, so + s * ld4);
    }
    __device__ void load_partial(int k0, int K, int h)
    {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int k = k0 + 2 * s + h;
            V x;
            __builtin_memcpy(&x, col + std::int64_t(k < K ? k : K - 1) * ld, sizeof(x));
            u[s] = k < K ? x : V{};
        }
    }
};

template <class Cfg, bool TA, bool TB, bool EDGE>
struct WsOps {
    using A = std::conditional_t<TA, WsFC<Cfg, EDGE>, WsKC<Cfg, EDGE>>;
    using B = std::conditional_t<TB, WsKC<Cfg, EDGE>, WsFC<Cfg, EDGE>>;
    static constexpr int kChunkLoads = A::kLoads + B::kLoads;  // vector loads of one chunk
};

template <int NB, int S, class OA, class OB>
__device__ __forceinline__ void ws_chunk(ws_f32x16 (&acc)[NB][NB], const OA &a, const OB &b)
{
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int t = 0; t < NB; ++t)
                acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.get(i, s), b.get(t, s), acc[i][t], 0, 0, 0);
}

// The first `steps` steps of a chunk (the partial one: its k order puts
// every k < K in the first ceil(rem / 2) steps).
template <int NB, int S, class OA, class OB>
__device__ __forceinline__ void ws_chunk_steps(ws_f32x16 (&acc)[NB][NB], const OA &a, const OB &b, int steps)
{
#pragma unroll
    for (int s = 0; s < S; ++s)
        if (s < steps)
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int t = 0; t < NB; ++t)
                    acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.get(i, s), b.get(t, s), acc[i][t], 0, 0, 0);
}

// One T x T tile (tm, tn); `red` holds Cfg::kRedFloats floats.
template <class Cfg, bool TA, bool TB, bool EDGE>
__device__ __forceinline__ void wsplit_tile(const Problem &p, int tm, int tn, float *red)
{
    using OA = typename WsOps<Cfg, TA, TB, EDGE>::A;
    using OB = typename WsOps<Cfg, TA, TB, EDGE>::B;
    constexpr int NB = Cfg::NB, S = Cfg::S, CH = Cfg::CH, SETS = Cfg::SETS, RR = Cfg::RR;
    const int lane = threadIdx.x % 64, l32 = lane % 32, h = lane / 32;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const std::int64_t m0 = std::int64_t(tm) * Cfg::T;
    const std::int64_t n0 = std::int64_t(tn) * Cfg::T;
    const int nfull = p.K / CH;
    // Chunks w, w + 4, w + 8, ... of the full ones belong to this wave.
    const int n = nfull > w ? (nfull - 1 - w) / kWsWaves + 1 : 0;

    ws_f32x16 acc[NB][NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int t = 0; t < NB; ++t) acc[i][t] = ws_f32x16{};

    OA fa[SETS];
    OB fb[SETS];
#pragma unroll
    for (int u = 0; u < SETS; ++u) {
        fa[u].init(p.A, p.lda, m0, p.M, l32, h);
        fb[u].init(p.B, p.ldb, n0, p.N, l32, h);
    }
    // The next chunk's loads spread over this one's MFMAs, one load per
    // kPer MFMAs, so they never issue as a burst that holds back the MFMAs (a
    // wave issues in order); the MFMAs left over follow.
    constexpr int kLoads = WsOps<Cfg, TA, TB, EDGE>::kChunkLoads;
    constexpr int kMfmas = NB * NB * S;
    constexpr int kPer = kMfmas / kLoads;
    static_assert(kPer >= 1, "a load per MFMA at most");
    auto interleave = [] {
#pragma unroll
        for (int q = 0; q < kLoads; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // VMEM read
            __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);  // MFMA
        }
        if constexpr (kMfmas - kPer * kLoads > 0)
            __builtin_amdgcn_sched_group_barrier(0x008, kMfmas - kPer * kLoads, 0);
    };
    auto chunk = [&](int i) { return w + kWsWaves * i; };
    // The partial last chunk of K (if any) goes to wave nfull % 4, which has
    // the fewest full chunks when nfull is not a multiple of 4, and is
    // multiplied after the full ones. (Read at the start instead, or while
    // the last full chunk is multiplied, it measured slower: the first put
    // 5-17% on every product, the second spilled into the edge tiles' loop.)
    const int rem = p.K - nfull * CH;
    const bool partial = rem > 0 && w == nfull % kWsWaves;
    if (n > 0) {
#pragma unroll
        for (int u = 0; u + 1 < SETS; ++u) {
            const int c = u < n ? u : n - 1;
            fa[u].load(chunk(c));
            fb[u].load(chunk(c));
        }
        int i = 0;
        // SETS chunks per pass so that the sets are constants. The loads
        // SETS - 1 chunks ahead are issued even past the wave's last chunk
        // (its last chunk again, never used): under a branch they would
        // leave the compiler's count of loads in flight to the path without
        // them.
        for (; i + SETS <= n; i += SETS) {
#pragma unroll
            for (int u = 0; u < SETS; ++u) {
                const int c = i + u + SETS - 1 < n ? i + u + SETS - 1 : n - 1;
                fa[(u + SETS - 1) % SETS].load(chunk(c));
                fb[(u + SETS - 1) % SETS].load(chunk(c));
                ws_chunk<NB, S>(acc, fa[u], fb[u]);
                interleave();
            }
        }
#pragma unroll
        for (int u = 0; u + 1 < SETS; ++u)
            if (i + u < n) ws_chunk<NB, S>(acc, fa[u], fb[u]);
    }
    if (partial) {
        fa[SETS - 1].load_partial(nfull * CH, p.K, h);
        fb[SETS - 1].load_partial(nfull * CH, p.K, h);
        ws_chunk_steps<NB, S>(acc, fa[SETS - 1], fb[SETS - 1], (rem + 1) / 2);
    }

    // The four partial tiles meet in LDS, RR block rows at a time. In a
    // round, quad q = ((a - a0) * NB + t) * 4 + g holds registers 4g .. 4g+3
    // of block (a, t), at red[((w * Q + q) * 64 + lane) * 4].
    constexpr int Q = RR * NB * 4;
#pragma unroll
    for (int a0 = 0; a0 < NB; a0 += RR) {
        if (a0 > 0) __syncthreads();  // the previous round's reads are done
#pragma unroll
        for (int a = a0; a < a0 + RR; ++a)
#pragma unroll
            for (int t = 0; t < NB; ++t)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const ws_f32x4 x = {acc[a][t][4 * g], acc[a][t][4 * g + 1], acc[a][t][4 * g + 2],
                                        acc[a][t][4 * g + 3]};
                    *reinterpret_cast<ws_f32x4 *>(&red[((w * Q + ((a - a0) * NB + t) * 4 + g) * 64 + lane) * 4]) =
                        x;
                }
        __syncthreads();
        // The round's RR x 4 (block row, register group) pairs, RR to a wave:
        // wave w takes pairs w RR .. w RR + RR - 1. It sums (partial 0 +
        // partial 1) + partial 2 + partial 3 for every block column.
        float sum[RR][NB][4];  // [pair][t][e]
#pragma unroll
        for (int k = 0; k < RR; ++k) {
            const int pi = w * RR + k, al = pi / 4, g = pi % 4;
#pragma unroll
            for (int t = 0; t < NB; ++t) {
                const int q = (al * NB + t) * 4 + g;
                ws_f32x4 s4 = *reinterpret_cast<const ws_f32x4 *>(&red[(q * 64 + lane) * 4]);
#pragma unroll
                for (int ww = 1; ww < kWsWaves; ++ww)
                    s4 += *reinterpret_cast<const ws_f32x4 *>(&red[((ww * Q + q) * 64 + lane) * 4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) sum[k][t][e] = s4[e];
            }
        }
        // Register r = 4g + e of block (a, t) is MFMA row 8g + 4h + e, column l32.
        auto c_row = [&](int k, int e) {
            const int pi = w * RR + k, al = pi / 4, g = pi % 4;
            return m0 + OA::free_index(a0 + al, 8 * g + 4 * h + e);
        };
        if constexpr (!TB && NB != 3) {
            // B as given: a lane's NB block columns are NB adjacent columns of C.
            const std::int64_t col = n0 + NB * l32;
            float old[RR][4][NB] = {};
            if (p.beta != 0.0f) {
#pragma unroll
                for (int k = 0; k < RR; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        read_c<NB>(p.C, p.ldc, c_row(k, e), int(col), p.M, p.N, !EDGE, old[k][e]);
            }
#pragma unroll
            for (int k = 0; k < RR; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v[NB];
#pragma unroll
                    for (int t = 0; t < NB; ++t) v[t] = sum[k][t][e];
                    write_c<NB>(p.C, p.ldc, c_row(k, e), int(col), p.M, p.N, v, old[k][e], !EDGE, p.alpha, p.beta);
                }
        } else {
            float old[RR][NB][4][1] = {};
            if (p.beta != 0.0f) {
#pragma unroll
                for (int k = 0; k < RR; ++k)
#pragma unroll
                    for (int t = 0; t < NB; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            read_c<1>(p.C, p.ldc, c_row(k, e), int(n0 + OB::free_index(t, l32)), p.M, p.N, !EDGE,
                                      old[k][t][e]);
            }
#pragma unroll
            for (int k = 0; k < RR; ++k)
#pragma unroll
                for (int t = 0; t < NB; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v[1] = {sum[k][t][e]};
                        write_c<1>(p.C, p.ldc, c_row(k, e), int(n0 + OB::free_index(t, l32)), p.M, p.N, v,
                                   old[k][t][e], !EDGE, p.alpha, p.beta);
                    }
        }
    }
}

template <class Cfg, bool TA, bool TB>
__global__ __launch_bounds__(64 * kWsWaves) __attribute__((amdgpu_waves_per_eu(Cfg::WPE, Cfg::WPE))) void
mfma_wsplit_kernel(Problem p, int tiles_m)
{
    __shared__ __attribute__((aligned(16))) float red[Cfg::kRedFloats];
    int tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, SGEMM_MFMA_GROUP_M, tm, tn);
    const bool edge = std::int64_t(tm + 1) * Cfg::T > p.M || std::int64_t(tn + 1) * Cfg::T > p.N;
    if (edge)
        wsplit_tile<Cfg, TA, TB, true>(p, tm, tn, red);
    else
        wsplit_tile<Cfg, TA, TB, false>(p, tm, tn, red);
}

// Whether every buffer offset of the product fits the 31 bits the kernel
// forms them in: for a KC operand, T rows from the tile's first one; for an
// FC operand, the whole stored matrix (K rows).
template <class Cfg>
bool wsplit_offsets_fit(const Problem &p)
{
    constexpr std::int64_t kLimit = std::int64_t(1) << 31;
    auto kc_fits = [&](std::int64_t ld) { return (std::int64_t(Cfg::T) * ld + p.K) * 4 < kLimit; };
    auto fc_fits = [&](std::int64_t ld, std::int64_t extent) { return (std::int64_t(p.K) * ld + extent) * 4 < kLimit; };
    const bool a_ok = p.ta ? fc_fits(p.lda, p.M) : kc_fits(p.lda);
    const bool b_ok = p.tb ? kc_fits(p.ldb) : fc_fits(p.ldb, p.N);
    return a_ok && b_ok;
}

template <class Cfg, bool TA, bool TB>
hipError_t launch_wsplit(const Problem &p, hipStream_t stream)
{
    const void *kernel = reinterpret_cast<const void *>(&mfma_wsplit_kernel<Cfg, TA, TB>);
    return for_each_band<Cfg::T, Cfg::T>(p, [&](Problem q, int tiles_m, int tiles_n) {
        void *args[] = {&q, &tiles_m};
        return hipLaunchKernel(kernel, dim3(unsigned(tiles_m) * unsigned(tiles_n)), dim3(64 * kWsWaves), args, 0,
                               stream);
    });
}

}  // namespace
}  // namespace sgemm_impl

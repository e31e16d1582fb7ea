// The matrix-core tile for products that give each compute unit about one
// 64 x 64 tile of C (1024^3 has 256 of them for 256 compute units): the
// work-group's four waves each compute the WHOLE 64 x 64 tile over a quarter
// of K, and the four partial tiles are summed at the end. Splitting K this
// way is free: the terms of a dot product may be added in any grouping
// ("Matrix Multiplication -- Naive to Tiled", section 07 on split-K), and
// here the grouping is fixed, so every run gives the same bits.
//
// Why not the LDS-staged loop of the other tiles: with one small tile per
// compute unit, each wave has one or two 32 x 32 blocks, and the loop spends
// its time on the barrier of every slab and the wait for the fragments read
// after it. Here a wave shares nothing with the others until the end, so the
// loop has no LDS and no barrier:
//  * a wave reads its operands straight from global memory (L2) into
//    registers, already in the order v_mfma_f32_32x32x2_f32 takes them, one
//    chunk of 32 k ahead of the one it multiplies (a chunk is 64 MFMAs, about
//    1.7 us: longer than a load's round trip);
//  * buffer loads carry the per-lane part of each address in one VGPR and the
//    per-row and per-chunk parts in scalar registers, so the loop issues no
//    vector address arithmetic between its MFMAs;
//  * chunk c belongs to wave c % 4; the partial tiles meet once, in LDS.
//
// K order inside a chunk of 32 (k0 .. k0+31): MFMA step s (0..15) gives lane
// half h the k index k0 + 16h + s. So
//  * an operand stored with k contiguous ("KC": A as given, B transposed)
//    gives lane (l32, h) of block b the 16 values X[f][k0+16h .. k0+16h+15]
//    of its free index f = 32b + l32 as four 16-byte loads;
//  * an operand stored with its free index contiguous ("FC": B as given, A
//    transposed) gives lane (c, h) the pair X[k0+16h+s][2c, 2c+1] with one
//    8-byte load per step; element e of the pair feeds block e, so block e
//    covers the free indices 2c + e and a lane ends up with two adjacent
//    columns of C (B as given), stored with one 8-byte access.
//
// Ragged shapes: a KC row past the operand's edge is read from the last row
// (its values only reach rows of C that are never stored); an FC pair that
// crosses the edge is read from the last two elements and shifted down by
// one, so the one valid element lands in its place. The partial last chunk
// of K (rem = K mod 32 values) is read element by element with zeros past K,
// in a k order of its own, k0 + 2s + h for step s and lane half h, so that
// its values fill the first ceil(rem / 2) steps and the rest are skipped.
// Its loads are not prefetched, so a ragged K costs each tile a load's round
// trip; the host takes this tile for ragged K only where a compute unit
// holds a single tile. This needs the FC operand at least 2 wide (narrower
// products take the general tiles).
#pragma once

#include <cstdint>
#include <type_traits>

#include "gemm.hpp"
#include "tile_io.hpp"

namespace sgemm_impl {
namespace {

typedef float ws_f32x16 __attribute__((ext_vector_type(16)));
typedef float ws_f32x4 __attribute__((ext_vector_type(4)));
typedef float ws_f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWsTile = 64;   // BM = BN
constexpr int kWsWaves = 4;   // K split over the work-group's waves
constexpr int kWsChunk = 32;  // k per chunk
// gfx9 buffer resource word 3 for untyped 32-bit accesses.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const float *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, 0x7fffffff, kBufferWord3);
}

// An operand stored with k contiguous. The resource starts at the tile's
// first free index; lane offsets are relative to it.
template <bool EDGE>
struct WsKC {
    ws_f32x4 v[2][4];  // v[b][j][e]: k = k0 + 16h + 4j + e of block b
    __amdgpu_buffer_rsrc_t rs;
    int vo[2];  // byte offset of (free index of block b, k = 16h)
    const float *row[2];  // the same rows as plain pointers (partial chunk)

    static constexpr int kLoads = 8;  // per chunk
    __device__ float get(int b, int s) const { return v[b][s / 4][s % 4]; }
    __device__ static int free_index(int b, int l32) { return 32 * b + l32; }

    __device__ void init(const float *X, std::int64_t ld, std::int64_t f0, std::int64_t extent, int l32, int h)
    {
        rs = ws_rsrc(X + f0 * ld);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            std::int64_t f = f0 + 32 * b + l32;
            if (EDGE && f >= extent) f = extent - 1;
            vo[b] = int(((f - f0) * ld + 16 * h) * 4);
            row[b] = X + f * ld;
        }
    }
    // Full chunk c (k0 = 32c).
    __device__ void load(int c)
    {
        const int so = c * kWsChunk * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                v[b][j] = __builtin_bit_cast(ws_f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo[b] + 16 * j, so, 0));
    }
    // The partial chunk starting at k0, in its own k order (step s, half h:
    // k = k0 + 2s + h), with zeros at k >= K.
    __device__ void load_partial(int k0, int K, int h)
    {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int k = k0 + 2 * s + h;
                const float x = row[b][k < K ? k : K - 1];
                v[b][s / 4][s % 4] = k < K ? x : 0.0f;
            }
    }
};

// An operand stored with its free index contiguous. The resource starts at
// the operand itself (free index 0), so that an edge pair can be read from
// the last two elements wherever the tile starts.
template <bool EDGE>
struct WsFC {
    ws_f32x2 u[16];  // u[s][e]: k = k0 + 16h + s, free index 2c + e
    __amdgpu_buffer_rsrc_t rs;
    int vo, ld4;
    bool shift;  // the pair was read one element early (edge): element 1 is the lane's
    const float *col;  // the lane's pair in stored row 0 (partial chunk)
    std::int64_t ld;

    static constexpr int kLoads = 16;  // per chunk
    // The shift is applied where a value is used, not where it is loaded: a
    // select right after the load would wait for the load there and then.
    __device__ float get(int b, int s) const
    {
        if constexpr (EDGE)
            if (b == 0) return shift ? u[s][1] : u[s][0];
        return u[s][b];
    }
    __device__ static int free_index(int b, int l32) { return 2 * l32 + b; }

    __device__ void init(const float *X, std::int64_t ld_, std::int64_t f0, std::int64_t extent, int l32, int h)
    {
        ld = ld_;
        rs = ws_rsrc(X);
        std::int64_t f = f0 + 2 * l32;
        shift = false;
        if (EDGE && f + 1 >= extent) {
            shift = f < extent;  // one valid element, read as the pair's second
            f = extent - 2;
        }
        vo = int((16 * h * ld + f) * 4);
        ld4 = int(ld * 4);
        col = X + f;
    }
    __device__ void load(int c)
    {
        const int so = c * kWsChunk * ld4;
#pragma unroll
        for (int s = 0; s < 16; ++s)
            u[s] = __builtin_bit_cast(ws_f32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, vo, so + s * ld4, 0));
    }
    __device__ void load_partial(int k0, int K, int h)
    {
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int k = k0 + 2 * s + h;
            ws_f32x2 x;
            __builtin_memcpy(&x, col + std::int64_t(k < K ? k : K - 1) * ld, sizeof(x));
            u[s] = k < K ? x : ws_f32x2{0.0f, 0.0f};
        }
    }
};

template <bool TA, bool TB, bool EDGE>
struct WsOps {
    using A = std::conditional_t<TA, WsFC<EDGE>, WsKC<EDGE>>;
    using B = std::conditional_t<TB, WsKC<EDGE>, WsFC<EDGE>>;
    static constexpr int kChunkLoads = A::kLoads + B::kLoads;  // vector loads of one chunk
};

template <class OA, class OB>
__device__ __forceinline__ void ws_chunk(ws_f32x16 (&acc)[2][2], const OA &a, const OB &b)
{
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.get(i, s), b.get(t, s), acc[i][t], 0, 0, 0);
}

// The first `steps` steps of a chunk (the partial one: its k order puts
// every k < K in the first ceil(rem / 2) steps).
template <class OA, class OB>
__device__ __forceinline__ void ws_chunk_steps(ws_f32x16 (&acc)[2][2], const OA &a, const OB &b, int steps)
{
#pragma unroll
    for (int s = 0; s < 16; ++s)
        if (s < steps)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.get(i, s), b.get(t, s), acc[i][t], 0, 0, 0);
}

// One 64 x 64 tile (tm, tn); `red` holds kWsWaves * 64 * 64 floats.
template <bool TA, bool TB, bool EDGE>
__device__ __forceinline__ void wsplit_tile(const Problem &p, int tm, int tn, float *red)
{
    using OA = typename WsOps<TA, TB, EDGE>::A;
    using OB = typename WsOps<TA, TB, EDGE>::B;
    const int lane = threadIdx.x % 64, l32 = lane % 32, h = lane / 32;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const std::int64_t m0 = std::int64_t(tm) * kWsTile;
    const std::int64_t n0 = std::int64_t(tn) * kWsTile;
    const int nfull = p.K / kWsChunk;
    // Chunks w, w + 4, w + 8, ... of the full ones belong to this wave.
    const int n = nfull > w ? (nfull - 1 - w) / kWsWaves + 1 : 0;

    ws_f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[i][t] = ws_f32x16{};

    OA fa[2];
    OB fb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        fa[u].init(p.A, p.lda, m0, p.M, l32, h);
        fb[u].init(p.B, p.ldb, n0, p.N, l32, h);
    }
    // The next chunk's loads (16, 24 or 32 with the transpose pair) spread
    // over the 64 MFMAs of this one, one load per 64 / kLoads MFMAs, so they
    // never issue as a burst that holds back the MFMAs (a wave issues in
    // order); the MFMAs left over follow.
    constexpr int kLoads = WsOps<TA, TB, EDGE>::kChunkLoads;
    constexpr int kPer = 64 / kLoads;
    auto interleave = [] {
#pragma unroll
        for (int q = 0; q < kLoads; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // VMEM read
            __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);  // MFMA
        }
        if constexpr (64 - kPer * kLoads > 0) __builtin_amdgcn_sched_group_barrier(0x008, 64 - kPer * kLoads, 0);
    };
    auto chunk = [&](int i) { return w + kWsWaves * i; };
    // The partial last chunk of K (if any) goes to wave nfull % 4, which has
    // the fewest full chunks when nfull is not a multiple of 4, and is
    // multiplied after the full ones. (Read at the start instead, or while
    // the last full chunk is multiplied, it measured slower: the first put
    // 5-17% on every product, the second spilled into the edge tiles' loop.)
    const int rem = p.K - nfull * kWsChunk;
    const bool partial = rem > 0 && w == nfull % kWsWaves;
    if (n > 0) {
        fa[0].load(chunk(0));
        fb[0].load(chunk(0));
        int i = 0;
        // Two chunks per pass so that the buffers are constants. The next
        // chunk's loads are issued even past the wave's last chunk (its last
        // chunk again, never used): under a branch they would leave the
        // compiler's count of loads in flight to the path without them.
        for (; i + 2 <= n; i += 2) {
            const int c1 = i + 1 < n ? i + 1 : n - 1;
            fa[1].load(chunk(c1));
            fb[1].load(chunk(c1));
            ws_chunk(acc, fa[0], fb[0]);
            interleave();
            const int c2 = i + 2 < n ? i + 2 : n - 1;
            fa[0].load(chunk(c2));
            fb[0].load(chunk(c2));
            ws_chunk(acc, fa[1], fb[1]);
            interleave();
        }
        if (i < n) ws_chunk(acc, fa[0], fb[0]);
    }
    if (partial) {
        fa[1].load_partial(nfull * kWsChunk, p.K, h);
        fb[1].load_partial(nfull * kWsChunk, p.K, h);
        ws_chunk_steps(acc, fa[1], fb[1], (rem + 1) / 2);
    }

    // The four partial tiles meet in LDS: quad q = (a * 2 + t) * 4 + g holds
    // registers 4g .. 4g+3 of block (a, t), at red[((w * 16 + q) * 64 + lane) * 4].
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const ws_f32x4 x = {acc[a][t][4 * g], acc[a][t][4 * g + 1], acc[a][t][4 * g + 2], acc[a][t][4 * g + 3]};
                *reinterpret_cast<ws_f32x4 *>(&red[((w * 16 + (a * 2 + t) * 4 + g) * 64 + lane) * 4]) = x;
            }
    __syncthreads();
    // Wave w sums (partial 0 + partial 1) + partial 2 + partial 3 for block
    // row a = w / 2, register groups g = 2 (w % 2) and 2 (w % 2) + 1, both
    // block columns: 32 of the tile's 4096 values per lane... 16 per pair of
    // adjacent columns when B is as given.
    const int a = w / 2;
    float sum[2][2][4];  // [gg][t][e]
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int q = (a * 2 + t) * 4 + 2 * (w % 2) + gg;
            ws_f32x4 s4 = *reinterpret_cast<const ws_f32x4 *>(&red[(q * 64 + lane) * 4]);
#pragma unroll
            for (int ww = 1; ww < kWsWaves; ++ww)
                s4 += *reinterpret_cast<const ws_f32x4 *>(&red[((ww * 16 + q) * 64 + lane) * 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[gg][t][e] = s4[e];
        }
    // Register r = 4g + e of block (a, t) is MFMA row 8g + 4h + e, column l32.
    auto c_row = [&](int gg, int e) {
        const int i = 8 * (2 * (w % 2) + gg) + 4 * h + e;
        return m0 + OA::free_index(a, i);
    };
    if constexpr (!TB) {
        // B as given: the two block columns are adjacent columns of C.
        const std::int64_t col = n0 + 2 * l32;
        float old[2][4][2] = {};
        if (p.beta != 0.0f) {
#pragma unroll
            for (int gg = 0; gg < 2; ++gg)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const std::int64_t row = c_row(gg, e);
                    read_c<2>(p.C, p.ldc, row, int(col), p.M, p.N, !EDGE, old[gg][e]);
                }
        }
#pragma unroll
        for (int gg = 0; gg < 2; ++gg)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const std::int64_t row = c_row(gg, e);
                const float v[2] = {sum[gg][0][e], sum[gg][1][e]};
                write_c<2>(p.C, p.ldc, row, int(col), p.M, p.N, v, old[gg][e], !EDGE, p.alpha, p.beta);
            }
    } else {
        float old[2][2][4][1] = {};
        if (p.beta != 0.0f) {
#pragma unroll
            for (int gg = 0; gg < 2; ++gg)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        read_c<1>(p.C, p.ldc, c_row(gg, e), int(n0 + OB::free_index(t, l32)), p.M, p.N, !EDGE,
                                  old[gg][t][e]);
        }
#pragma unroll
        for (int gg = 0; gg < 2; ++gg)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v[1] = {sum[gg][t][e]};
                    write_c<1>(p.C, p.ldc, c_row(gg, e), int(n0 + OB::free_index(t, l32)), p.M, p.N, v,
                               old[gg][t][e], !EDGE, p.alpha, p.beta);
                }
    }
}

template <bool TA, bool TB>
__global__ __launch_bounds__(64 * kWsWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_wsplit_kernel(
    Problem p, int tiles_m)
{
    __shared__ __attribute__((aligned(16))) float red[kWsWaves * kWsTile * kWsTile];
    int tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, SGEMM_MFMA_GROUP_M, tm, tn);
    const bool edge = std::int64_t(tm + 1) * kWsTile > p.M || std::int64_t(tn + 1) * kWsTile > p.N;
    if (edge)
        wsplit_tile<TA, TB, true>(p, tm, tn, red);
    else
        wsplit_tile<TA, TB, false>(p, tm, tn, red);
}

// Whether every buffer offset of the product fits the 31 bits the kernel
// forms them in: for a KC operand, 64 rows from the tile's first one; for an
// FC operand, the whole stored matrix (K rows).
inline bool wsplit_offsets_fit(const Problem &p)
{
    constexpr std::int64_t kLimit = std::int64_t(1) << 31;
    auto kc_fits = [&](std::int64_t ld) { return (std::int64_t(kWsTile) * ld + p.K) * 4 < kLimit; };
    auto fc_fits = [&](std::int64_t ld, std::int64_t extent) { return (std::int64_t(p.K) * ld + extent) * 4 < kLimit; };
    const bool a_ok = p.ta ? fc_fits(p.lda, p.M) : kc_fits(p.lda);
    const bool b_ok = p.tb ? kc_fits(p.ldb) : fc_fits(p.ldb, p.N);
    return a_ok && b_ok;
}

template <bool TA, bool TB>
hipError_t launch_wsplit(const Problem &p, hipStream_t stream)
{
    const void *kernel = reinterpret_cast<const void *>(&mfma_wsplit_kernel<TA, TB>);
    return for_each_band<kWsTile, kWsTile>(p, [&](Problem q, int tiles_m, int tiles_n) {
        void *args[] = {&q, &tiles_m};
        return hipLaunchKernel(kernel, dim3(unsigned(tiles_m) * unsigned(tiles_n)), dim3(64 * kWsWaves), args, 0,
                               stream);
    });
}

}  // namespace
}  // namespace sgemm_impl

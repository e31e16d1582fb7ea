// Rung 3: register blocking on the vector ALUs ("Matrix Multiplication --
// Naive to Tiled", section 07: register tiling, double buffering, vectorised
// loads; "From 306 ms to 86 ms", "Register blocking"; "Shared Memory Tiling
// for Matrix Multiplication", traps: bank conflicts), extended to
// C = alpha * op(A) * op(B) + beta * C.
//
// A 256-work-item group owns a BM x BN tile of C and walks K in slabs of BK;
// each work-item keeps a TM x TN block of C in registers. The pages' tile is
// 128 x 128 with 8 x 8 per work-item: per k it reads 8 values of A and 8 of B
// from LDS with four 16-byte reads and does 64 multiply-adds, where the tiled
// rung did 1 multiply-add per 2 LDS reads. Products with too few of those
// tiles to occupy the chip take 64 x 64 tiles (4 x 4 per work-item), 32 x 32
// tiles (2 x 2) or, for the smallest, 16 x 16 tiles (1 x 1, slabs of 64),
// with the same loop.
//
// Layout and scheduling:
//  * the work-item (tx, ty) of a 16 x 16 grid owns rows VM*ty .. VM*ty+VM-1
//    of each TM/VM strips of 16*VM rows (VM = min(TM, 4)), and the same
//    pattern of columns with tx; for 8 x 8 these are rows {4ty..4ty+3,
//    64+4ty..64+4ty+3}. Every LDS read of a wave64 then stays inside one
//    contiguous span (no bank conflicts, broadcasts across the wave);
//  * both tiles are stored k-major in LDS, so the values a work-item needs at
//    one k are contiguous: op(A) is transposed on the way in when A is given
//    M x K and copied as is when A is given transposed; op(B) is copied as is
//    when B is given K x N and transposed on the way in when B is given
//    transposed; rows carry 4 words of padding;
//  * each work-item moves one 16-byte chunk of each operand per slab (BK is
//    chosen so that a slab of either operand is 256 chunks). Slab t+1 is
//    fetched into registers while slab t is multiplied out of LDS, then
//    written to the other of two LDS buffers, so one barrier per slab
//    suffices;
//  * elements outside A, B or C read as 0 / are not written (ragged shapes).
//
// The product is formed with scalar v_fma_f32 only (packed FP32 is disabled
// for this library), so this rung's ceiling is half the chip's FP32 peak.
#include "gemm.hpp"
#include "select.hpp"
#include "tile_io.hpp"

namespace sgemm_impl {
namespace {

constexpr int kThreads = 256;
constexpr int kPad = 4;
constexpr int kGroupM = 8;

template <int BM_, int BN_, int BK_>
struct RbConfig {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int TM = BM / 16, TN = BN / 16;             // C block per work-item
    static constexpr int VM = TM < 4 ? TM : 4, VN = TN < 4 ? TN : 4;  // floats per LDS read
    static constexpr int HM = TM / VM, HN = TN / VN;             // strips, 16 * V rows apart
    static_assert(BM * BK == 4 * kThreads && BN * BK == 4 * kThreads, "one chunk of each operand per work-item");
    static_assert(TM * VM > 0 && TM % VM == 0 && TN % VN == 0, "whole strips");
};

template <int V>
struct RbVec;
template <>
struct RbVec<1> {
    typedef float type;
};
template <>
struct RbVec<4> {
    typedef float4 type;
};
template <>
struct RbVec<2> {
    typedef float2 type;
};

template <int V>
__device__ __forceinline__ void rb_read(float *dst, const float *src)
{
    const typename RbVec<V>::type v = *reinterpret_cast<const typename RbVec<V>::type *>(src);
    if constexpr (V == 4) {
        dst[0] = v.x;
        dst[1] = v.y;
        dst[2] = v.z;
        dst[3] = v.w;
    } else if constexpr (V == 2) {
        dst[0] = v.x;
        dst[1] = v.y;
    } else {
        dst[0] = v;
    }
}

template <class Cfg, bool TA, bool TB, bool VEC>
__global__ __launch_bounds__(kThreads) void regblock_kernel(Problem p, int tiles_m)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, TM = Cfg::TM, TN = Cfg::TN;
    constexpr int VM = Cfg::VM, VN = Cfg::VN;
    __shared__ __attribute__((aligned(16))) float As[2][BK][BM + kPad];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK][BN + kPad];

    int tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, kGroupM, tm, tn);
    const std::int64_t m0 = std::int64_t(tm) * BM;
    const int n0 = tn * BN;

    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;

    // Global -> LDS assignment: one 4-wide chunk of op(A) and one of op(B)
    // per slab, taken along the operand's stored rows. A tile stored M x K:
    // BM rows of BK / 4 chunks of k; stored K x M: BK rows of BM / 4 chunks
    // of m (B likewise with N).
    const int a_f = TA ? (tid % (BM / 4)) * 4 : tid / (BK / 4);  // free index (m) of the chunk's first element
    const int a_k = TA ? tid / (BM / 4) : (tid % (BK / 4)) * 4;  // k of the chunk's first element
    const int b_f = TB ? tid / (BK / 4) : (tid % (BN / 4)) * 4;
    const int b_k = TB ? (tid % (BK / 4)) * 4 : tid / (BN / 4);

    const bool rows_in = m0 + BM <= p.M;
    const bool cols_in = n0 + BN <= p.N;
    const int n_slabs = (p.K + BK - 1) / BK;

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

    auto fetch = [&](int slab, float4 &ra, float4 &rb) {
        const int k0 = slab * BK;
        const bool k_in = k0 + BK <= p.K;
        if constexpr (TA)
            ra = load4<VEC>(p.A, p.lda, k0 + a_k, int(m0) + a_f, p.K, p.M, rows_in && k_in);
        else
            ra = load4<VEC>(p.A, p.lda, m0 + a_f, k0 + a_k, p.M, p.K, rows_in && k_in);
        if constexpr (TB)
            rb = load4<VEC>(p.B, p.ldb, n0 + b_f, k0 + b_k, p.N, p.K, k_in && cols_in);
        else
            rb = load4<VEC>(p.B, p.ldb, k0 + b_k, n0 + b_f, p.K, p.N, k_in && cols_in);
    };
    auto stash = [&](int buf, const float4 &ra, const float4 &rb) {
        if constexpr (TA) {
            *reinterpret_cast<float4 *>(&As[buf][a_k][a_f]) = ra;
        } else {
            As[buf][a_k + 0][a_f] = ra.x;
            As[buf][a_k + 1][a_f] = ra.y;
            As[buf][a_k + 2][a_f] = ra.z;
            As[buf][a_k + 3][a_f] = ra.w;
        }
        if constexpr (TB) {
            Bs[buf][b_k + 0][b_f] = rb.x;
            Bs[buf][b_k + 1][b_f] = rb.y;
            Bs[buf][b_k + 2][b_f] = rb.z;
            Bs[buf][b_k + 3][b_f] = rb.w;
        } else {
            *reinterpret_cast<float4 *>(&Bs[buf][b_k][b_f]) = rb;
        }
    };

    if (n_slabs > 0) {
        float4 ra, rb;
        fetch(0, ra, rb);
        stash(0, ra, rb);
        __syncthreads();
        for (int t = 0; t < n_slabs; ++t) {
            const int cur = t & 1;
            const bool more = t + 1 < n_slabs;
            if (more) fetch(t + 1, ra, rb);
#pragma unroll
            for (int k = 0; k < BK; ++k) {
                float a[TM], b[TN];
#pragma unroll
                for (int h = 0; h < Cfg::HM; ++h) rb_read<VM>(a + h * VM, &As[cur][k][h * 16 * VM + VM * ty]);
#pragma unroll
                for (int h = 0; h < Cfg::HN; ++h) rb_read<VN>(b + h * VN, &Bs[cur][k][h * 16 * VN + VN * tx]);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
            }
            if (more) stash(cur ^ 1, ra, rb);
            __syncthreads();
        }
    }

    // Epilogue: row strip i / VM, row VM*ty + i % VM in it; columns likewise
    // in strips of VN.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const std::int64_t row = m0 + (i / VM) * 16 * VM + VM * ty + i % VM;
#pragma unroll
        for (int h = 0; h < Cfg::HN; ++h) {
            float v[VN];
#pragma unroll
            for (int e = 0; e < VN; ++e) v[e] = acc[i][h * VN + e];
            const int c = n0 + h * 16 * VN + VN * tx;
            update_n<VN>(p.C, p.ldc, row, c, p.M, p.N, v, row < p.M && c + VN <= p.N, p.alpha, p.beta);
        }
    }
}

using RbLarge = RbConfig<128, 128, 8>;  // the pages' tile: 8 x 8 per work-item
using RbMid = RbConfig<64, 64, 16>;     // 4 x 4
using RbSmall = RbConfig<32, 32, 32>;   // 2 x 2
using RbTiny = RbConfig<16, 16, 64>;    // 1 x 1

template <class Cfg, bool TA, bool TB>
hipError_t launch(const Problem &p, hipStream_t stream)
{
    const void *kernel = rows_aligned16(p) ? reinterpret_cast<const void *>(&regblock_kernel<Cfg, TA, TB, true>)
                                           : reinterpret_cast<const void *>(&regblock_kernel<Cfg, TA, TB, false>);
    return for_each_band<Cfg::BM, Cfg::BN>(p, [&](Problem q, int tiles_m, int tiles_n) {
        void *args[] = {&q, &tiles_m};
        return hipLaunchKernel(kernel, dim3(unsigned(tiles_m) * unsigned(tiles_n)), dim3(kThreads), args, 0, stream);
    });
}

template <class Cfg>
hipError_t launch_cfg(const Problem &p, hipStream_t stream)
{
    if (p.ta) return p.tb ? launch<Cfg, true, true>(p, stream) : launch<Cfg, true, false>(p, stream);
    return p.tb ? launch<Cfg, false, true>(p, stream) : launch<Cfg, false, false>(p, stream);
}

}  // namespace

hipError_t launch_regblock(const Problem &p, hipStream_t stream)
{
    switch (regblock_tile_size(p.M, p.N, p.cus)) {
    case 16: return launch_cfg<RbTiny>(p, stream);
    case 32: return launch_cfg<RbSmall>(p, stream);
    case 64: return launch_cfg<RbMid>(p, stream);
    default: return launch_cfg<RbLarge>(p, stream);
    }
}

}  // namespace sgemm_impl

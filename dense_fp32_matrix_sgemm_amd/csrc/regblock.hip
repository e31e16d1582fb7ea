// Rung 3: register blocking on the vector ALUs ("Matrix Multiplication --
// Naive to Tiled", section 07: register tiling, double buffering, vectorised
// loads; "From 306 ms to 86 ms", "Register blocking"; "Shared Memory Tiling
// for Matrix Multiplication", traps: bank conflicts), extended to
// C = alpha * op(A) * op(B) + beta * C.
//
// A 256-work-item group owns a 128 x 128 tile of C and walks K in slabs of 8.
// Each work-item keeps an 8 x 8 block of C in registers: per k it reads 8
// values of A and 8 of B from LDS with four 16-byte reads and does 64
// multiply-adds, where the tiled rung did 1 multiply-add per 2 LDS reads.
//
// Layout and scheduling:
//  * the work-item (tx, ty) of a 16 x 16 grid owns rows {4ty..4ty+3,
//    64+4ty..64+4ty+3} and the same pattern of columns with tx; the two
//    4-wide halves 64 apart keep every LDS read of a wave64 inside one
//    contiguous span (no bank conflicts, broadcasts across the wave);
//  * both tiles are stored k-major in LDS, so the 8 rows (columns) a
//    work-item needs at one k are contiguous: op(A) is transposed on the way
//    in when A is given M x K and copied as is when A is given transposed;
//    op(B) is copied as is when B is given K x N and transposed on the way in
//    when B is given transposed; rows carry 4 words of padding;
//  * slab t+1 is fetched from global memory into registers with 16-byte loads
//    while slab t is multiplied out of LDS, then written to the other of two
//    LDS buffers, so one barrier per slab suffices;
//  * elements outside A, B or C read as 0 / are not written (ragged shapes).
//
// The product is formed with scalar v_fma_f32 only (packed FP32 is disabled
// for this library), so this rung's ceiling is half the chip's FP32 peak.
#include "gemm.hpp"
#include "tile_io.hpp"

namespace sgemm_impl {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 8;
constexpr int kTM = 8, kTN = 8;
constexpr int kThreads = (kBM / kTM) * (kBN / kTN);  // 256
constexpr int kPad = 4;
constexpr int kGroupM = 8;

template <bool TA, bool TB, bool VEC>
__global__ __launch_bounds__(kThreads) void regblock_kernel(Problem p, int tiles_m)
{
    __shared__ __attribute__((aligned(16))) float As[2][kBK][kBM + kPad];
    __shared__ __attribute__((aligned(16))) float Bs[2][kBK][kBN + kPad];

    int tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, kGroupM, tm, tn);
    const std::int64_t m0 = std::int64_t(tm) * kBM;
    const int n0 = tn * kBN;

    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;

    // Global -> LDS assignment: one 4-wide chunk of op(A) and one of op(B)
    // per slab, taken along the operand's stored rows. A tile stored M x K:
    // 128 rows x 2 chunks of k; stored K x M: 8 rows x 32 chunks of m (B
    // likewise with N).
    const int a_f = TA ? (tid % 32) * 4 : tid / 2;  // free index (m) of the chunk's first element
    const int a_k = TA ? tid / 32 : (tid % 2) * 4;  // k of the chunk's first element
    const int b_f = TB ? tid / 2 : (tid % 32) * 4;
    const int b_k = TB ? (tid % 2) * 4 : tid / 32;

    const bool rows_in = m0 + kBM <= p.M;
    const bool cols_in = n0 + kBN <= p.N;
    const int n_slabs = (p.K + kBK - 1) / kBK;

    float acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = 0.0f;

    auto fetch = [&](int slab, float4 &ra, float4 &rb) {
        const int k0 = slab * kBK;
        const bool k_in = k0 + kBK <= p.K;
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
            for (int k = 0; k < kBK; ++k) {
                const float4 a0 = *reinterpret_cast<const float4 *>(&As[cur][k][4 * ty]);
                const float4 a1 = *reinterpret_cast<const float4 *>(&As[cur][k][64 + 4 * ty]);
                const float4 b0 = *reinterpret_cast<const float4 *>(&Bs[cur][k][4 * tx]);
                const float4 b1 = *reinterpret_cast<const float4 *>(&Bs[cur][k][64 + 4 * tx]);
                const float a[kTM] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                const float b[kTN] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                for (int i = 0; i < kTM; ++i)
#pragma unroll
                    for (int j = 0; j < kTN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
            }
            if (more) stash(cur ^ 1, ra, rb);
            __syncthreads();
        }
    }

    // Epilogue: rows 4ty+i (i < 4) and 64+4ty+(i-4); columns likewise.
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        const std::int64_t row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + (i - 4));
        const float lo[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
        const float hi[4] = {acc[i][4], acc[i][5], acc[i][6], acc[i][7]};
        const int c_lo = n0 + 4 * tx, c_hi = n0 + 64 + 4 * tx;
        update_n<4>(p.C, p.ldc, row, c_lo, p.M, p.N, lo, row < p.M && c_lo + 4 <= p.N, p.alpha, p.beta);
        update_n<4>(p.C, p.ldc, row, c_hi, p.M, p.N, hi, row < p.M && c_hi + 4 <= p.N, p.alpha, p.beta);
    }
}

template <bool TA, bool TB>
hipError_t launch(const Problem &p, hipStream_t stream)
{
    const void *kernel = rows_aligned16(p) ? reinterpret_cast<const void *>(&regblock_kernel<TA, TB, true>)
                                           : reinterpret_cast<const void *>(&regblock_kernel<TA, TB, false>);
    return for_each_band<kBM, kBN>(p, [&](Problem q, int tiles_m, int tiles_n) {
        void *args[] = {&q, &tiles_m};
        return hipLaunchKernel(kernel, dim3(unsigned(tiles_m) * unsigned(tiles_n)), dim3(kThreads), args, 0, stream);
    });
}

}  // namespace

hipError_t launch_regblock(const Problem &p, hipStream_t stream)
{
    if (p.ta) return p.tb ? launch<true, true>(p, stream) : launch<true, false>(p, stream);
    return p.tb ? launch<false, true>(p, stream) : launch<false, false>(p, stream);
}

}  // namespace sgemm_impl

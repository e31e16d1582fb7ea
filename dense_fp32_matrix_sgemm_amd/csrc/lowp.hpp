// The reduced-precision workload: C = alpha * op(A) * op(B) + beta * C with A
// and B given as bf16 or f16 and every product summed in FP32, on the gfx950
// matrix cores (v_mfma_f32_32x32x16_bf16 / _f16). This is the tensor-core
// variant "Matrix Multiplication -- Naive to Tiled", section 07 names (FP16 in,
// FP32 accumulate), on CDNA's matrix cores. Each dtype is its own translation
// unit (lowp_bf16.hip, lowp_f16.hip).
//
// The tile hierarchy is the FP32 kernel's (mfma.hpp): a work-group owns a
// BM x BN tile of C and walks K in slabs of BK through two LDS buffers, one
// barrier per slab, with slab t+1 staged in registers while slab t is
// multiplied. What changes with 16-bit operands:
//  * v_mfma_f32_32x32x16: lane l supplies 8 consecutive k of its operand's
//    free index l % 32 (k = 8 (l / 32) + 0..7 within the instruction's 16);
//    the accumulator layout is that of the FP32 instruction.
//  * So every lane needs 8 k at one free index. A tile stored with k
//    contiguous ("KC": A as given, B transposed) gives them with one 16-byte
//    LDS read (rows padded by 8 elements, which puts the 16 rows a quarter-wave
//    reads in distinct banks).
//  * A tile stored with its free index contiguous ("FC": B as given, A
//    transposed) stays in that order in LDS, so global memory still moves to
//    LDS in 16-byte chunks; the transpose happens in the read, with gfx950's
//    ds_read_b64_tr_b16: within each group of 16 lanes, lanes 4r..4r+3 name
//    the 16 consecutive elements of row r (4 each) and lane i receives element
//    i of rows 0..3. Two such reads (rows k..k+3 and k+4..k+7) give a lane its
//    8 values. FC rows are padded by 32 elements so the 8 rows a pass touches
//    fall in distinct banks.
//  * Both read orders give lane half h the k indices 8h + 0..7 of each step of
//    16, so any pairing of KC and FC operands sums the same terms.
//
// Edge tiles run the same loop with their reads clamped into the operands (a
// KC row past the edge reads the last row; an FC chunk crossing the edge reads
// the last 8 elements of its row and is shifted into place when stored to LDS;
// junk only reaches rows or columns of C that are never stored); a partial
// last slab of K is loaded element by element with zeros past K. This needs
// the FC operand at least 8 wide; narrower products take a one-thread-per-
// element kernel.
//
// Products large enough for one 256 x 256 tile per compute unit, with
// 16-byte aligned rows, take a second kernel (lp_dma_tile below): four waves
// of 128 x 128, operands moved global -> LDS by DMA through four swizzled
// stages. Both kernels read the same k order per lane, so a product gives the
// same terms in the same order whichever of them runs.
#pragma once

#include <type_traits>

#include "gemm.hpp"
#include "tile_io.hpp"

namespace sgemm_impl {
namespace {

typedef float lp_f32x16 __attribute__((ext_vector_type(16)));
typedef short lp_i16x8 __attribute__((ext_vector_type(8)));
typedef short lp_i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 lp_f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 lp_bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) lp_i16x4 lp_lds_i16x4;

template <LpType T>
__device__ __forceinline__ lp_f32x16 mma16(lp_i16x8 a, lp_i16x8 b, lp_f32x16 c)
{
    if constexpr (T == LpType::BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(lp_bf16x8, a),
                                                        __builtin_bit_cast(lp_bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(lp_f16x8, a),
                                                       __builtin_bit_cast(lp_f16x8, b), c, 0, 0, 0);
}

// Exact float value of one 16-bit encoding.
template <LpType T>
__device__ __forceinline__ float widen(std::uint16_t v)
{
    if constexpr (T == LpType::BF16) {
        return __uint_as_float(std::uint32_t(v) << 16);
    } else {
        return float(__builtin_bit_cast(_Float16, v));
    }
}

__device__ __forceinline__ lp_i16x8 load16u_i16(const std::uint16_t *p)
{
    lp_i16x8 v;
    __builtin_memcpy(&v, p, sizeof(v));
    return v;
}

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct LpConfig {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int kGroupM = 8;
    static constexpr int kAccRegs = (WM / 32) * (WN / 32) * 16;
    static constexpr int kWavesPerEU = kAccRegs >= 256 ? 1 : kAccRegs >= 64 ? 2 : 4;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK % 16 == 0, "slab depth must be whole steps of 16");
};

// One operand's share of a work-group tile: F free indices by BK values of k,
// W free indices per wave, copied by NT work-items in 16-byte chunks (8
// elements). In LDS (one stage, in elements):
//   KC: F rows of BK values, padded by 8:   lds[f * (BK + 8) + k];
//   FC: BK rows of F values, padded by 32:  lds[k * (F + 32) + f].
template <int F, int W, int BK, int NT, bool KC_>
struct LpOperand {
    static constexpr bool KC = KC_;
    static constexpr int NB = W / 32;                      // MFMA blocks per wave
    static constexpr int kPitch = KC ? BK + 8 : F + 32;
    static constexpr int kRows = KC ? F : BK;              // stored rows in a tile
    static constexpr int kRowLen = KC ? BK : F;
    static constexpr int kElems = kRows * kPitch;
    static constexpr int kRowChunks = kRowLen / 8;
    static constexpr int kChunks = F * BK / 8 / NT;        // chunks per work-item per slab
    static constexpr int kRowStep = NT / kRowChunks;       // stored rows between them
    static constexpr int kReads = KC ? NB : 2 * NB;        // LDS reads per step of 16 k
    static_assert(kChunks >= 1 && kChunks * 8 * NT == F * BK, "tile must split evenly over the work-items");
    static_assert(NT % kRowChunks == 0, "chunk rows must advance evenly");

    __device__ static constexpr int chunk_row(int c) { return c / kRowChunks; }
    __device__ static constexpr int chunk_col(int c) { return (c % kRowChunks) * 8; }
    __device__ static constexpr int chunk_lds(int c) { return chunk_row(c) * kPitch + chunk_col(c); }

    // Operand values of one step of 16 k: v[b] feeds block b.
    struct Frag {
        lp_i16x8 v[NB];
    };

    // Fragments of step s of the stage at `lds` for the wave whose free
    // indices start at w0.
    __device__ static void read(Frag &fr, const short *lds, int w0, int s, int lane)
    {
        if constexpr (KC) {
            const int l32 = lane % 32, h = lane / 32;
#pragma unroll
            for (int b = 0; b < NB; ++b)
                fr.v[b] = *reinterpret_cast<const lp_i16x8 *>(&lds[(w0 + b * 32 + l32) * kPitch + 16 * s + 8 * h]);
        } else {
            // Lane 4r + q of a 16-lane group names row k0 + r, elements
            // 4q .. 4q+3 of the group's 16 columns; it receives its own column.
            const int g = lane / 16, i = lane % 16, r = i / 4, q = i % 4;
            const int k0 = 16 * s + 8 * (g / 2) + r;
            const int f = w0 + 16 * (g % 2) + 4 * q;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const short *p0 = &lds[k0 * kPitch + f + 32 * b];
                const lp_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp_lds_i16x4 *)(p0));
                const lp_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp_lds_i16x4 *)(p0 + 4 * kPitch));
                fr.v[b] = lp_i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        }
    }
};

// Where one work-item's chunks of an operand tile come from: chunk q of every
// slab starts at chunk(q) + slab offset. With EDGE the addresses are clamped
// into the operand and place() shifts an FC chunk read from a moved address
// back into place.
template <class Op, bool EDGE>
struct LpSource {
    const std::uint16_t *base;
    std::int64_t ld;
    std::int64_t off[EDGE && Op::KC ? Op::kChunks : 1];
    int shift;  // FC: elements the read was moved left

    __device__ LpSource(const std::uint16_t *X, std::int64_t ld_, std::int64_t f0, std::int64_t extent, int tid)
        : base(X), ld(ld_), shift(0)
    {
        const int r0 = Op::chunk_row(tid), c0 = Op::chunk_col(tid);
        if constexpr (Op::KC) {
            if constexpr (EDGE) {
#pragma unroll
                for (int q = 0; q < Op::kChunks; ++q) {
                    const std::int64_t f = f0 + r0 + q * Op::kRowStep;
                    off[q] = (f < extent ? f : extent - 1) * ld + c0;
                }
            } else {
                off[0] = (f0 + r0) * ld + c0;
            }
        } else {
            std::int64_t f = f0 + c0;
            if constexpr (EDGE) {
                const std::int64_t last = extent - 8;  // extent >= 8
                const std::int64_t fr = f < last ? f : last;
                const std::int64_t d = f - fr;
                shift = int(d < 7 ? d : 7);
                f = fr;
            }
            off[0] = std::int64_t(r0) * ld + f;
        }
    }
    __device__ const std::uint16_t *chunk(int q) const
    {
        if constexpr (EDGE && Op::KC)
            return base + off[q];
        else
            return base + off[0] + std::int64_t(q) * Op::kRowStep * ld;
    }
    // Element e of the chunk is element e + shift of what was read.
    __device__ lp_i16x8 place(lp_i16x8 v) const
    {
        if constexpr (EDGE && !Op::KC) {
            unsigned __int128 x = __builtin_bit_cast(unsigned __int128, v);
            x >>= 16 * shift;
            return __builtin_bit_cast(lp_i16x8, x);
        } else {
            return v;
        }
    }
};

constexpr int kLpSchedMfma = 0x008, kLpSchedVmemRead = 0x020, kLpSchedDsRead = 0x100, kLpSchedDsWrite = 0x200;

// One BM x BN tile (tm, tn); `lds` holds two stages of both operand tiles.
template <class Cfg, LpType T, bool TA, bool TB, bool EDGE>
__device__ __forceinline__ void lp_tile(const LpProblem &p, int tm, int tn, short *lds)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::kThreads;
    using OpA = LpOperand<BM, Cfg::WM, BK, NT, !TA>;
    using OpB = LpOperand<BN, Cfg::WN, BK, NT, TB>;
    constexpr int G = BK / 16;  // steps of 16 k per slab
    // The steady loop reads the next slab's step 0 into fragment slot 0 before
    // it multiplies this slab's last step from slot (G - 1) & 1: an even G.
    static_assert(G % 2 == 0, "the pipelined slab loop needs an even number of steps of 16 k");
    constexpr int CA = OpA::kChunks, CB = OpB::kChunks;
    constexpr int NA = OpA::NB, NBl = OpB::NB;

    short(*As)[OpA::kElems] = reinterpret_cast<short(*)[OpA::kElems]>(lds);
    short(*Bs)[OpB::kElems] = reinterpret_cast<short(*)[OpB::kElems]>(lds + 2 * OpA::kElems);

    const std::int64_t m0 = std::int64_t(tm) * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wm0 = (wave / Cfg::WAVES_N) * Cfg::WM;
    const int wn0 = (wave % Cfg::WAVES_N) * Cfg::WN;
    const int n_full = p.K / BK;

    lp_f32x16 acc[NA][NBl];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < NBl; ++b) acc[a][b] = lp_f32x16{};

    const LpSource<OpA, EDGE> srca(p.A, p.lda, m0, p.M, tid);
    const LpSource<OpB, EDGE> srcb(p.B, p.ldb, n0, p.N, tid);
    const std::int64_t slab_a = OpA::KC ? BK : BK * p.lda, slab_b = OpB::KC ? BK : BK * p.ldb;

    lp_i16x8 ra[CA], rb[CB];
    auto fetch = [&](int slab) {
        const std::int64_t ka = slab * slab_a, kb = slab * slab_b;
#pragma unroll
        for (int q = 0; q < CA; ++q) ra[q] = load16u_i16(srca.chunk(q) + ka);
#pragma unroll
        for (int q = 0; q < CB; ++q) rb[q] = load16u_i16(srcb.chunk(q) + kb);
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int q = 0; q < CA; ++q)
            *reinterpret_cast<lp_i16x8 *>(&As[buf][OpA::chunk_lds(q * NT + tid)]) = srca.place(ra[q]);
#pragma unroll
        for (int q = 0; q < CB; ++q)
            *reinterpret_cast<lp_i16x8 *>(&Bs[buf][OpB::chunk_lds(q * NT + tid)]) = srcb.place(rb[q]);
    };

    typename OpA::Frag fa[2];
    typename OpB::Frag fb[2];
    auto read_frags = [&](int buf, int s, int slot) {
        OpA::read(fa[slot], As[buf], wm0, s, lane);
        OpB::read(fb[slot], Bs[buf], wn0, s, lane);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int b = 0; b < NBl; ++b) acc[a][b] = mma16<T>(fa[slot].v[a], fb[slot].v[b], acc[a][b]);
    };
    auto multiply = [&](int buf) {
        read_frags(buf, 0, 0);
#pragma unroll
        for (int s = 0; s < G; ++s) {
            if (s + 1 < G) read_frags(buf, s + 1, (s + 1) & 1);
            mfmas(s & 1);
        }
    };

    // Interleave hints for a slab: its fragment reads, LDS stores and global
    // loads spread evenly over the MFMAs of all but its last step (a wave
    // issues in order, so a burst of memory instructions would hold back the
    // next MFMA).
    constexpr int NR = OpA::kReads + OpB::kReads;
    constexpr int kMf = (G - 1) * NA * NBl;
    constexpr int kMem = (G - 1) * NR + 2 * (CA + CB);
    constexpr int kPer = (kMem + kMf - 1) / kMf;  // memory instructions after each MFMA
    auto interleave = [&] {
        constexpr int R = (G - 1) * NR, W = CA + CB, L = CA + CB;
#pragma unroll
        for (int i = 0; i < kMf; ++i) {
            __builtin_amdgcn_sched_group_barrier(kLpSchedMfma, 1, 0);
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int m = i * kPer + j;  // memory instruction number, reads first
                if (m < R)
                    __builtin_amdgcn_sched_group_barrier(kLpSchedDsRead, 1, 0);
                else if (m < R + W)
                    __builtin_amdgcn_sched_group_barrier(kLpSchedDsWrite, 1, 0);
                else if (m < R + W + L)
                    __builtin_amdgcn_sched_group_barrier(kLpSchedVmemRead, 1, 0);
            }
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
        // Steady state (as in the FP32 kernel): store slab t+1 to the other
        // buffer, start loading slab t+2, multiply steps 0..G-2 of slab t while
        // reading steps 1..G-1; barrier; read step 0 of slab t+1 while
        // multiplying step G-1 of slab t.
        for (; t + 2 < n; ++t) {
            const int cur = t & 1;
            stash(cur ^ 1);
            fetch(t + 2);
#pragma unroll
            for (int s = 0; s + 1 < G; ++s) {
                read_frags(cur, s + 1, (s + 1) & 1);
                mfmas(s & 1);
            }
            interleave();
            __syncthreads();
            read_frags(cur ^ 1, 0, 0);
            mfmas((G - 1) & 1);
        }
        for (; t < n; ++t) {
            const int cur = t & 1;
            if (t + 1 < n) stash(cur ^ 1);
#pragma unroll
            for (int s = 0; s + 1 < G; ++s) {
                read_frags(cur, s + 1, (s + 1) & 1);
                mfmas(s & 1);
            }
            __syncthreads();
            if (t + 1 < n) read_frags(cur ^ 1, 0, 0);
            mfmas((G - 1) & 1);
        }
        __syncthreads();
    }
    if (n_full * BK < p.K) {
        // Partial last slab: k >= K reads as zero, free indices past the
        // operand's extent are clamped into it.
        const int k0 = n_full * BK;
        auto partial = [&](auto op, const std::uint16_t *X, std::int64_t ld, std::int64_t f0, std::int64_t extent,
                           short *dst) {
            using Op = decltype(op);
            // All of this work-item's loads first, then the LDS stores, so
            // that the loads are in flight together.
            constexpr int kPer = Op::kRows * Op::kRowLen / NT;
            static_assert(kPer * NT == Op::kRows * Op::kRowLen, "whole elements per work-item");
            short v[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int e = tid + i * NT;
                const int r = e / Op::kRowLen, c = e % Op::kRowLen;
                const int k = Op::KC ? c : r;
                const std::int64_t f = f0 + (Op::KC ? r : c);
                const std::int64_t fc = f < extent ? f : extent - 1;
                const std::int64_t at = Op::KC ? fc * ld + k0 + k : std::int64_t(k0 + k) * ld + fc;
                v[i] = k0 + k < p.K ? short(X[at]) : short(0);
            }
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int e = tid + i * NT;
                dst[(e / Op::kRowLen) * Op::kPitch + e % Op::kRowLen] = v[i];
            }
        };
        partial(OpA{}, p.A, p.lda, m0, p.M, As[0]);
        partial(OpB{}, p.B, p.ldb, n0, p.N, Bs[0]);
        __syncthreads();
        multiply(0);
    }

    // Epilogue: register r of block (a, b) is row 32a + 8(r/4) + 4h + r%4 and
    // column 32b + l % 32 of the wave tile. With beta != 0 a block's 16 old
    // values of C are read before any of them is written, so that the reads
    // are in flight together.
    const int l32 = lane % 32, h = lane / 32;
    auto row_of = [&](int a, int r) -> std::int64_t { return m0 + wm0 + 32 * a + 8 * (r / 4) + 4 * h + (r % 4); };
    if (p.beta != 0.0f) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int b = 0; b < NBl; ++b) {
                const int col = n0 + wn0 + 32 * b + l32;
                float old[16][1];
#pragma unroll
                for (int r = 0; r < 16; ++r) read_c<1>(p.C, p.ldc, row_of(a, r), col, p.M, p.N, !EDGE, old[r]);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float v[1] = {acc[a][b][r]};
                    write_c<1>(p.C, p.ldc, row_of(a, r), col, p.M, p.N, v, old[r], !EDGE, p.alpha, p.beta);
                }
            }
        return;
    }
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
            for (int b = 0; b < NBl; ++b) {
                const float v[1] = {acc[a][b][r]};
                update_n<1>(p.C, p.ldc, row_of(a, r), n0 + wn0 + 32 * b + l32, p.M, p.N, v, !EDGE, p.alpha, p.beta);
            }
        }
}

template <class Cfg, bool TA, bool TB>
constexpr int lp_lds_elems()
{
    return 2 * (LpOperand<Cfg::BM, Cfg::WM, Cfg::BK, Cfg::kThreads, !TA>::kElems +
                LpOperand<Cfg::BN, Cfg::WN, Cfg::BK, Cfg::kThreads, TB>::kElems);
}

// Waves per SIMD a work-group of this kernel can have resident: the tile's
// register budget (Cfg::kWavesPerEU), or fewer where its two LDS stages
// leave room for fewer work-groups in a compute unit's 160 KiB.
template <class Cfg, bool TA, bool TB>
constexpr int lp_waves_per_eu()
{
    constexpr int kLdsPerCu = 160 * 1024;
    constexpr int wg_per_cu = kLdsPerCu / (int(sizeof(short)) * lp_lds_elems<Cfg, TA, TB>());
    constexpr int by_lds = wg_per_cu * (Cfg::kThreads / 64) / 4;
    return by_lds < 1 ? 1 : by_lds < Cfg::kWavesPerEU ? by_lds : Cfg::kWavesPerEU;
}

template <class Cfg, LpType T, bool TA, bool TB>
__global__ __launch_bounds__(Cfg::kThreads)
__attribute__((amdgpu_waves_per_eu(lp_waves_per_eu<Cfg, TA, TB>(), lp_waves_per_eu<Cfg, TA, TB>()))) void lp_tiles_kernel(LpProblem p, int tiles_m)
{
    __shared__ __attribute__((aligned(16))) short lds[lp_lds_elems<Cfg, TA, TB>()];
    int tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, Cfg::kGroupM, tm, tn);
    const bool edge = std::int64_t(tm + 1) * Cfg::BM > p.M || std::int64_t(tn + 1) * Cfg::BN > p.N;
    if (edge)
        lp_tile<Cfg, T, TA, TB, true>(p, tm, tn, lds);
    else
        lp_tile<Cfg, T, TA, TB, false>(p, tm, tn, lds);
}

// Direct-to-LDS pipeline for large products.
//
// The loop above moves every slab global -> registers -> LDS, and a slab's
// loads have one slab of MFMAs to arrive. With 16-bit operands the matrix
// cores finish a slab 8 times sooner, relative to the bytes it moves, than in
// FP32, and that loop leaves them waiting on load latency and LDS bandwidth.
// This one differs in four ways:
//  * four waves (2 x 2) each multiply a 128 x 128 block of the 256 x 256
//    tile (16 accumulator blocks, one wave per SIMD): per slab the waves read
//    2/3 of the LDS bytes that eight 64 x 128 waves read;
//  * chunks go straight from global memory into LDS (global_load_lds_dwordx4:
//    one instruction writes 64 consecutive 16-byte chunks) through S stages:
//    slab t + S - 1 is requested while slab t is multiplied, so a load has
//    S - 2 slabs of MFMAs to arrive, with no staging registers and no LDS
//    store instructions;
//  * the DMA cannot pad rows, so instead the chunks of a stored row are
//    permuted (an XOR swizzle chosen through which global chunk each lane
//    fetches): KC rows of BK = 32 values hold chunk c at position
//    c ^ g(r), g(r) = ((r >> 1) + (r >> 3)) & 3; FC rows of F values hold
//    chunk j at position j ^ h(k), h(k) = ((k & 3) << 2) ^ (k & 2). With
//    these the lanes of a ds_read_b128 or ds_read_b64_tr_b16 that the LDS
//    serves together fall in distinct banks, for 32 four-byte banks serving
//    128 bytes per cycle and for 64 serving 256;
//  * the accumulators leave through LDS (the stages are free by then), so
//    that every store writes 512 contiguous bytes of each of two rows of C.
// A barrier per slab publishes the next stage (each wave first waits for its
// own DMA of it, with the s_waitcnt count of the loads it may leave in
// flight) and frees the stage the DMA issued after it overwrites. The
// barrier is written out rather than taken from __syncthreads, whose fence
// would wait for every load in flight, the later stages' included.
//
// Requirements (checked by the host): 16-byte aligned operands with leading
// dimensions that are multiples of 8 elements, and an FC extent (N with B as
// given, M with A transposed) that is a multiple of 8, so no chunk straddles
// the edge. Edge tiles read clamped rows (KC) or the last chunk (FC) past the
// edge; those values reach only rows and columns of C that are not stored. A
// partial last slab of K is filled element by element with zeros past K.
template <int F, int BK, bool KC_>
struct LpDmaOperand {
    static constexpr bool KC = KC_;
    static constexpr int kRowChunks = KC ? BK / 8 : F / 8;  // chunks per stored row
    static constexpr int kRowLen = KC ? BK : F;             // elements per stored row
    static constexpr int kRows = KC ? F : BK;               // stored rows per slab
    static constexpr int kElems = F * BK;                   // one stage
    static constexpr int kInstrs = F * BK / 8 / 64;         // DMA instructions per slab
    static_assert(BK == 32, "the KC swizzle is for rows of 4 chunks");
    static_assert(KC || (F >= 128 && (F & (F - 1)) == 0), "the FC swizzle needs rows of 16 or more chunks");

    __host__ __device__ static constexpr int swz(int row)
    {
        return KC ? (((row >> 1) + (row >> 3)) & 3) : (((row & 3) << 2) ^ (row & 2));
    }
    // Element offset, in one stage, of chunk c of stored row r.
    __host__ __device__ static constexpr int lds_of(int r, int c) { return (r * kRowChunks + (c ^ swz(r))) * 8; }
};

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct LpDmaConfig : LpConfig<BM_, BN_, BK_, WAVES_M_, WAVES_N_> {
    static constexpr int kStages = STAGES_;
    static_assert(STAGES_ >= 3, "the DMA of slab t + S - 1 reuses the stage of slab t - 1");
};

// LDS byte address of a location in a __shared__ array.
__device__ __forceinline__ unsigned lp_lds_address(const short *p)
{
    return static_cast<unsigned>(reinterpret_cast<std::uintptr_t>((const __attribute__((address_space(3))) short *)p));
}

// One global_load_lds_dwordx4: lane i copies the 16 bytes at its src to LDS
// byte address lds + 16 i (lds is wave-uniform; the instruction takes it in
// M0, which the compiler loads for the statement as its input operand).
// Written as inline assembly so that the compiler does not see an LDS store
// whose completion it would then wait for (with vmcnt(0)) before LDS reads
// of other stages; the loop's own waits order it.
__device__ __forceinline__ void lp_dma16(const std::uint16_t *src, unsigned lds)
{
    asm volatile("global_load_lds_dwordx4 %1, off" ::"{m0}"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
                 : "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0), then s_barrier; also a compiler barrier for
// memory accesses.
template <int N>
__device__ __forceinline__ void lp_wait_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <class Cfg, LpType T, bool TA, bool TB>
__device__ __forceinline__ void lp_dma_tile(const LpProblem &p, int tm, int tn, short *lds)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, S = Cfg::kStages;
    constexpr int NW = Cfg::WAVES_M * Cfg::WAVES_N;
    using OpA = LpDmaOperand<BM, BK, !TA>;
    using OpB = LpDmaOperand<BN, BK, TB>;
    constexpr int NA = Cfg::WM / 32, NBl = Cfg::WN / 32;
    constexpr int CA = OpA::kInstrs / NW, CB = OpB::kInstrs / NW;  // DMA instructions per wave per slab
    constexpr int kStage = OpA::kElems + OpB::kElems;
    constexpr int kPerSlab = CA + CB;
    static_assert(CA * NW == OpA::kInstrs && CB * NW == OpB::kInstrs, "DMA must split evenly over the waves");
    static_assert(BK == 32, "two steps of 16 k per slab");

    const std::int64_t m0 = std::int64_t(tm) * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wm0 = (wave / Cfg::WAVES_N) * Cfg::WM;
    const int wn0 = (wave % Cfg::WAVES_N) * Cfg::WN;
    const int n = p.K / BK;

    lp_f32x16 acc[NA][NBl];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < NBl; ++b) acc[a][b] = lp_f32x16{};

    // Global element offset, from the slab's start, of the chunk this lane
    // moves with DMA instruction q of an operand (instruction q * NW + wave
    // of the slab; its lanes fill 64 consecutive chunk positions).
    auto dma_offset = [&](auto op, int q, std::int64_t ld, std::int64_t f0, std::int64_t extent) -> std::int64_t {
        using Op = decltype(op);
        const int pos = (q * NW + wave) * 64 + lane;
        const int r = pos / Op::kRowChunks;
        const int c = (pos % Op::kRowChunks) ^ Op::swz(r);
        if constexpr (Op::KC) {
            std::int64_t f = f0 + r;
            f = f < extent ? f : extent - 1;
            return f * ld + 8 * c;
        } else {
            std::int64_t f = f0 + 8 * c;
            f = f < extent ? f : extent - 8;
            return std::int64_t(r) * ld + f;
        }
    };
    const std::uint16_t *srca[CA];
    const std::uint16_t *srcb[CB];
#pragma unroll
    for (int q = 0; q < CA; ++q) srca[q] = p.A + dma_offset(OpA{}, q, p.lda, m0, p.M);
#pragma unroll
    for (int q = 0; q < CB; ++q) srcb[q] = p.B + dma_offset(OpB{}, q, p.ldb, n0, p.N);
    const std::int64_t slab_a = OpA::KC ? BK : BK * p.lda, slab_b = OpB::KC ? BK : BK * p.ldb;

    auto stage_a = [&](int st) { return lds + st * kStage; };
    auto stage_b = [&](int st) { return lds + st * kStage + OpA::kElems; };
    // DMA instruction i (0 .. kPerSlab - 1) of slab `slab` into stage st:
    // the A instructions first, then the B ones.
    const unsigned lds_bytes = lp_lds_address(lds);
    auto dma_one = [&](int i, int slab, int st) {
        if (i < CA)
            lp_dma16(srca[i] + slab * slab_a, lds_bytes + 2u * unsigned(st * kStage + (i * NW + wave) * 512));
        else
            lp_dma16(srcb[i - CA] + slab * slab_b,
                     lds_bytes + 2u * unsigned(st * kStage + OpA::kElems + ((i - CA) * NW + wave) * 512));
    };

    // Per-lane fragment offsets within a stage, for step s of block b.
    const int l32 = lane % 32, h = lane / 32;
    auto frag_offsets = [&](auto op, int w0, int (&off)[2][4]) {
        using Op = decltype(op);
        if constexpr (Op::KC) {
            // Row w0 + 32 b + l32, chunk 2 s + h.
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int b = 0; b < 4; ++b) off[s][b] = Op::lds_of(w0 + 32 * b + l32, 2 * s + h);
        } else {
            // Lane 4 r + q of 16-lane group g: row 16 s + 8 (g / 2) + r,
            // elements w0 + 32 b + 16 (g % 2) + 4 q .. + 3.
            const int g = lane / 16, i = lane % 16, r = i / 4, q = i % 4;
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int k = 16 * s + 8 * (g / 2) + r;
                    const int f = w0 + 32 * b + 16 * (g % 2) + 4 * q;
                    off[s][b] = Op::lds_of(k, f / 8) + f % 8;
                }
        }
    };
    static_assert(NA == 4 && NBl == 4, "offset tables hold four blocks");
    int offa[2][4], offb[2][4];
    frag_offsets(OpA{}, wm0, offa);
    frag_offsets(OpB{}, wn0, offb);

    auto read_op = [&](auto op, lp_i16x8 &v, const short *stage, int o) {
        using Op = decltype(op);
        if constexpr (Op::KC) {
            v = *reinterpret_cast<const lp_i16x8 *>(stage + o);
        } else {
            const lp_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp_lds_i16x4 *)(stage + o));
            const lp_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp_lds_i16x4 *)(stage + o + 4 * Op::kRowLen));
            v = lp_i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    // Fragments of step s, block u (A blocks, then B blocks), into slot `slot`.
    lp_i16x8 fa[2][NA], fb[2][NBl];
    constexpr int NU = NA + NBl;
    auto read_unit = [&](int u, int st, int s, int slot) {
        if (u < NA)
            read_op(OpA{}, fa[slot][u], stage_a(st), offa[s][u]);
        else
            read_op(OpB{}, fb[slot][u - NA], stage_b(st), offb[s][u - NA]);
    };
    // The instruction takes B's fragment as its first operand and A's as its
    // second, and so computes the transpose of block (a, b): lane l holds
    // row l % 32 of the block and, in registers 4q .. 4q + 3, its columns
    // 8q + 4h .. 8q + 4h + 3. The fragments are the same either way (both
    // operands take 8 k of one free index per lane), and so are the sums.
    auto mfma_one = [&](int slot, int i) {
        const int a = i / NBl, b = i % NBl;
        acc[a][b] = mma16<T>(fb[slot][b], fa[slot][a], acc[a][b]);
    };

    // One step's MFMAs with the fragment reads for the other slot spread one
    // after each of the first MFMAs (so reads neither hold back an MFMA nor
    // wait until the MFMAs that need them), and DMA instructions d0 .. d0 +
    // nd - 1 of a slab spread evenly over the step (each is its own
    // scheduling region, which keeps the order as written).
    constexpr int kReads = (OpA::KC ? NA : 2 * NA) + (OpB::KC ? NBl : 2 * NBl);
    constexpr int kMfmas = NA * NBl;
    static_assert(kReads <= kMfmas && NU <= kMfmas && kPerSlab <= kMfmas, "one read and one DMA per MFMA at most");
    auto step = [&](int slot, int rd_st, int rd_s, bool reads, int dma_slab, int dma_st, int d0, int nd) {
#pragma unroll
        for (int i = 0; i < kMfmas; ++i) {
            if (nd > 0 && i % (kMfmas / nd) == 0 && i / (kMfmas / nd) < nd)
                dma_one(d0 + i / (kMfmas / nd), dma_slab, dma_st);
            mfma_one(slot, i);
            if (reads && i < NU) read_unit(i, rd_st, rd_s, slot ^ 1);
        }
#pragma unroll
        for (int i = 0; i < kMfmas; ++i) {
            __builtin_amdgcn_sched_group_barrier(kLpSchedMfma, 1, 0);
            if (reads && i < kReads) __builtin_amdgcn_sched_group_barrier(kLpSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    if (n > 0) {
        // Slab indices past the last are clamped to it: the loop then issues
        // the same DMA every iteration (the repeats land in the stage that is
        // free anyway), waits with one count, and has no branches, which
        // keeps the 256 accumulator registers where they are.
        auto last = [&](int slab) { return slab < n ? slab : n - 1; };
#pragma unroll
        for (int i = 0; i < S - 1; ++i)
#pragma unroll
            for (int d = 0; d < kPerSlab; ++d) dma_one(d, last(i), i);
        lp_wait_barrier<(S - 2) * kPerSlab>();
#pragma unroll
        for (int u = 0; u < NU; ++u) read_unit(u, 0, 0, 0);
        // Slab t + S - 1 goes into the stage slab t - 1 used, which the
        // barrier before step 0 of slab t frees: its first kEarly DMA
        // instructions go out during step 0, the rest during step 1, so the
        // two steps carry equal LDS traffic. Step 0 of slab t multiplies
        // while step 1's fragments load; slab t + 1 is published (slabs
        // t + 2 .. t + S - 2 and the early part of t + S - 1 may still be in
        // flight); step 1 multiplies while slab t + 1's first fragments load
        // (in the last iteration, from a stage nobody uses again).
#if defined(SGEMM_LP_DMA_EARLY)
        constexpr int kEarly = SGEMM_LP_DMA_EARLY;
#else
        constexpr int kEarly = kPerSlab / 2;
#endif
        static_assert(kEarly >= 0 && kEarly <= kPerSlab, "a split of the slab's DMA instructions");
        for (int t = 0; t < n; ++t) {
            const int dma_st = (t + S - 1) % S, dma_slab = last(t + S - 1);
            step(0, t % S, 1, true, dma_slab, dma_st, 0, kEarly);
            lp_wait_barrier<(S - 3) * kPerSlab + kEarly>();
            step(1, (t + 1) % S, 0, true, dma_slab, dma_st, kEarly, kPerSlab - kEarly);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the repeated DMAs
    }
    if (n * BK < p.K) {
        // Partial last slab into stage 0: k >= K reads as zero, free indices
        // past the operand's extent are clamped into it.
        lp_wait_barrier<0>();
        const int k0 = n * BK;
        auto partial = [&](auto op, const std::uint16_t *X, std::int64_t ld, std::int64_t f0, std::int64_t extent,
                           short *dst) {
            using Op = decltype(op);
            // All of this work-item's loads first, then the LDS stores, so
            // that the loads are in flight together.
            constexpr int kPer = Op::kRows * Op::kRowLen / Cfg::kThreads;
            static_assert(kPer * Cfg::kThreads == Op::kRows * Op::kRowLen, "whole elements per work-item");
            short v[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int e = tid + i * Cfg::kThreads;
                const int r = e / Op::kRowLen, c = e % Op::kRowLen;
                const int k = Op::KC ? c : r;
                const std::int64_t f = f0 + (Op::KC ? r : c);
                const std::int64_t fc = f < extent ? f : extent - 1;
                const std::int64_t at = Op::KC ? fc * ld + k0 + k : std::int64_t(k0 + k) * ld + fc;
                v[i] = k0 + k < p.K ? short(X[at]) : short(0);
            }
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int e = tid + i * Cfg::kThreads;
                const int r = e / Op::kRowLen, c = e % Op::kRowLen;
                dst[Op::lds_of(r, c / 8) + c % 8] = v[i];
            }
        };
        partial(OpA{}, p.A, p.lda, m0, p.M, stage_a(0));
        partial(OpB{}, p.B, p.ldb, n0, p.N, stage_b(0));
        lp_wait_barrier<0>();
#pragma unroll
        for (int u = 0; u < NU; ++u) read_unit(u, 0, 0, 0);
        step(0, 0, 1, true, 0, 0, 0, 0);
        step(1, 0, 0, false, 0, 0, 0, 0);
    }

    // Epilogue through LDS, one block row (32 rows of the wave tile) at a
    // time: each lane writes its 4-column pieces (register r of block (a, b)
    // is row 32a + l % 32, column 32b + 8(r/4) + 4h + r%4), then reads back 4
    // consecutive columns of a row, so that one store covers two rows of 512
    // contiguous bytes. (Stored straight from the accumulators, one store
    // covers 32 bytes of each of 32 rows, which is slow when the rows are a
    // large power of two apart.) Rows are padded by 4 floats, which puts the
    // 16 lanes an LDS pass serves in distinct banks for the writes and the
    // reads. Every wave stages in its own 32-row region; the barrier first
    // makes sure that no DMA or fragment read still uses the stages.
    const bool inside = m0 + BM <= p.M && n0 + BN <= p.N;
    constexpr int kPitch = Cfg::WN + 4;
    static_assert(NW * 32 * kPitch * 2 <= S * kStage, "staging fits in the operand stages");
    lp_wait_barrier<0>();
    float *stage_c = reinterpret_cast<float *>(lds) + wave * 32 * kPitch;
#pragma unroll
    for (int a = 0; a < NA; ++a) {
#pragma unroll
        for (int b = 0; b < NBl; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<f32x4u *>(stage_c + l32 * kPitch + 32 * b + 8 * q + 4 * h) =
                    f32x4u{acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]};
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's writes before its reads
        // With beta != 0 the 16 runs' old values of C are read first, so that
        // the reads are in flight together.
        float old[16][4];
        if (p.beta != 0.0f) {
#pragma unroll
            for (int it = 0; it < 16; ++it)
                read_c<4>(p.C, p.ldc, m0 + wm0 + 32 * a + 2 * it + h, n0 + wn0 + 4 * l32, p.M, p.N, inside, old[it]);
        }
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int row = 2 * it + h;
            const f32x4u x = *reinterpret_cast<const f32x4u *>(stage_c + row * kPitch + 4 * l32);
            const float v[4] = {x[0], x[1], x[2], x[3]};
            if (p.beta != 0.0f)
                write_c<4>(p.C, p.ldc, m0 + wm0 + 32 * a + row, n0 + wn0 + 4 * l32, p.M, p.N, v, old[it], inside,
                           p.alpha, p.beta);
            else
                update_n<4>(p.C, p.ldc, m0 + wm0 + 32 * a + row, n0 + wn0 + 4 * l32, p.M, p.N, v, inside, p.alpha,
                            p.beta);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reads before the next block row's writes
    }
}

template <class Cfg, LpType T, bool TA, bool TB>
__global__ __launch_bounds__(Cfg::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void lp_dma_kernel(
    LpProblem p, int tiles_m)
{
    __shared__ __attribute__((aligned(16))) short lds[Cfg::kStages * (Cfg::BM + Cfg::BN) * Cfg::BK];
    int tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, Cfg::kGroupM, tm, tn);
    lp_dma_tile<Cfg, T, TA, TB>(p, tm, tn, lds);
}

// Products whose FC operand is under 8 wide: one work-item per element of C,
// products of the widened values summed with FP32 fused multiply-adds.
template <LpType T, bool TA, bool TB>
__global__ __launch_bounds__(256) void lp_naive_kernel(LpProblem p)
{
    const int j = blockIdx.x * 64 + threadIdx.x;
    if (j >= p.N) return;
    const std::int64_t sa = TA ? p.lda : 1, sb = TB ? 1 : p.ldb;
    const std::uint16_t *b = TB ? p.B + std::int64_t(j) * p.ldb : p.B + j;
    for (std::int64_t i = std::int64_t(blockIdx.y) * 4 + threadIdx.y; i < p.M; i += std::int64_t(gridDim.y) * 4) {
        const std::uint16_t *a = TA ? p.A + i : p.A + i * p.lda;
        float acc = 0.0f;
        for (int k = 0; k < p.K; ++k) acc = __builtin_fmaf(widen<T>(a[k * sa]), widen<T>(b[k * sb]), acc);
        float *c = p.C + i * p.ldc + j;
        *c = p.beta != 0.0f ? axpby(p.alpha, acc, p.beta, *c) : p.alpha * acc;
    }
}

// Tile grids beyond 2^22 tiles run as bands (row bands of op(A) and C,
// column bands of op(B) and C), as the FP32 launches do.
template <class Cfg, LpType T, bool TA, bool TB, bool DMA = false>
hipError_t lp_launch_tiles(const LpProblem &p, hipStream_t stream)
{
    constexpr std::int64_t kMaxTiles = std::int64_t(1) << 22;
    const std::int64_t tiles_n_all = (std::int64_t(p.N) + Cfg::BN - 1) / Cfg::BN;
    const std::int64_t band_tn = tiles_n_all < kMaxTiles ? tiles_n_all : kMaxTiles;
    const std::int64_t band_tm = kMaxTiles / band_tn;
    const void *kernel;
    if constexpr (DMA)
        kernel = reinterpret_cast<const void *>(&lp_dma_kernel<Cfg, T, TA, TB>);
    else
        kernel = reinterpret_cast<const void *>(&lp_tiles_kernel<Cfg, T, TA, TB>);
    for (std::int64_t r0 = 0; r0 < p.M; r0 += band_tm * Cfg::BM) {
        for (std::int64_t c0 = 0; c0 < p.N; c0 += band_tn * Cfg::BN) {
            LpProblem q = p;
            q.M = int(p.M - r0 < band_tm * Cfg::BM ? p.M - r0 : band_tm * Cfg::BM);
            q.N = int(p.N - c0 < band_tn * Cfg::BN ? p.N - c0 : band_tn * Cfg::BN);
            q.A = TA ? p.A + r0 : p.A + r0 * p.lda;
            q.B = TB ? p.B + c0 * p.ldb : p.B + c0;
            q.C = p.C + r0 * p.ldc + c0;
            int tiles_m = int((q.M + Cfg::BM - 1) / Cfg::BM);
            const unsigned n_wg = unsigned(tiles_m) * unsigned((q.N + Cfg::BN - 1) / Cfg::BN);
            void *args[] = {&q, &tiles_m};
            const hipError_t e = hipLaunchKernel(kernel, dim3(n_wg), dim3(Cfg::kThreads), args, 0, stream);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

#ifndef SGEMM_LP_BIG_TILE
#define SGEMM_LP_BIG_TILE 256, 256, 32, 4, 2
#endif
#ifndef SGEMM_LP_MID_TILE
#define SGEMM_LP_MID_TILE 128, 128, 64, 4, 2
#endif
// 192 x 128 tiles (2 x 4 waves of 96 x 32) for products whose 128 x 128 tiles
// would leave the compute units unevenly loaded but whose 192 x 128 tiles take
// fewer rounds (3001 x 2047 takes 16 x 16 of them, one per compute unit,
// against 1.5 per compute unit of 128 x 128). With A stored M x K only: the
// 192-row tile of a transposed A is 24 chunks a row, which the work-items do
// not split evenly.
#ifndef SGEMM_LP_WIDE_TILE
#define SGEMM_LP_WIDE_TILE 192, 128, 64, 2, 4
#endif
// The 64x64 tile takes slabs of 64: against 32, +6% at 1024^3 and 1536^3 in
// an interleaved A/B (the 128x128 tile lost 7-16% with 32 instead of 64).
#ifndef SGEMM_LP_SMALL_TILE
#define SGEMM_LP_SMALL_TILE 64, 64, 64, 2, 2
#endif
#ifndef SGEMM_LP_DMA_TILE
#define SGEMM_LP_DMA_TILE 256, 256, 32, 2, 2, 4
#endif
using LpDmaCfg = LpDmaConfig<SGEMM_LP_DMA_TILE>;
using LpBigCfg = LpConfig<SGEMM_LP_BIG_TILE>;
using LpMidCfg = LpConfig<SGEMM_LP_MID_TILE>;
using LpWideCfg = LpConfig<SGEMM_LP_WIDE_TILE>;
using LpSmallCfg = LpConfig<SGEMM_LP_SMALL_TILE>;

template <class Cfg>
std::int64_t lp_tiles(const LpProblem &p)
{
    return ((std::int64_t(p.M) + Cfg::BM - 1) / Cfg::BM) * ((std::int64_t(p.N) + Cfg::BN - 1) / Cfg::BN);
}

// Whether the direct-to-LDS kernel can take a product: 16-byte aligned
// operands and rows, and an FC extent that is a multiple of 8.
template <bool TA, bool TB>
bool lp_dma_ok(const LpProblem &p)
{
#if defined(SGEMM_LP_NO_DMA)
    return false;
#else
    const auto aligned = [](const void *x) { return (reinterpret_cast<std::uintptr_t>(x) & 15) == 0; };
    return aligned(p.A) && aligned(p.B) && p.lda % 8 == 0 && p.ldb % 8 == 0 && (!TA || p.M % 8 == 0) &&
           (TB || p.N % 8 == 0);
#endif
}

// The largest tile shape whose tiles give every compute unit at least one;
// 192 x 128 instead of 128 x 128 where its rounds of one tile per compute
// unit cover less area.
template <LpType T, bool TA, bool TB>
hipError_t lp_launch(const LpProblem &p, hipStream_t stream)
{
    if ((TA && p.M < 8) || (!TB && p.N < 8)) {
        LpProblem q = p;
        void *args[] = {&q};
        const unsigned gy = unsigned((std::int64_t(p.M) + 3) / 4);
        return hipLaunchKernel(reinterpret_cast<const void *>(&lp_naive_kernel<T, TA, TB>),
                               dim3(unsigned((p.N + 63) / 64), gy < kMaxGridY ? gy : kMaxGridY), dim3(64, 4), args,
                               0, stream);
    }
    const std::int64_t fill = p.cus > 0 ? p.cus : 256;
    if (lp_tiles<LpDmaCfg>(p) >= fill && lp_dma_ok<TA, TB>(p)) return lp_launch_tiles<LpDmaCfg, T, TA, TB, true>(p, stream);
    if (lp_tiles<LpBigCfg>(p) >= fill) return lp_launch_tiles<LpBigCfg, T, TA, TB>(p, stream);
    if constexpr (!TA) {
        // Rounds of one tile per compute unit, times the tile's area.
        const auto area = [&](std::int64_t tiles, std::int64_t bm, std::int64_t bn) {
            return (tiles + fill - 1) / fill * bm * bn;
        };
        const std::int64_t mid = lp_tiles<LpMidCfg>(p);
        if (mid >= fill && area(lp_tiles<LpWideCfg>(p), LpWideCfg::BM, LpWideCfg::BN) <
                               area(mid, LpMidCfg::BM, LpMidCfg::BN))
            return lp_launch_tiles<LpWideCfg, T, TA, TB>(p, stream);
    }
    if (lp_tiles<LpMidCfg>(p) >= fill) return lp_launch_tiles<LpMidCfg, T, TA, TB>(p, stream);
    return lp_launch_tiles<LpSmallCfg, T, TA, TB>(p, stream);
}

// Dispatch on the transpose pair.
template <LpType T>
hipError_t lp_launch_any(const LpProblem &p, hipStream_t stream)
{
    if (p.ta) return p.tb ? lp_launch<T, true, true>(p, stream) : lp_launch<T, true, false>(p, stream);
    return p.tb ? lp_launch<T, false, true>(p, stream) : lp_launch<T, false, false>(p, stream);
}

}  // namespace
}  // namespace sgemm_impl

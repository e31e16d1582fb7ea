// Rung 4: the LDS-tiled, double-buffered product fed to the CDNA matrix cores
// with v_mfma_f32_32x32x2_f32 (FP32 operands, FP32 accumulation). The pages'
// kernels stop at register blocking on CUDA cores ("Matrix Multiplication --
// Naive to Tiled", section 07, which names tensor-core MMA only for FP16
// inputs); on gfx950 the FP32 dense contraction itself has a matrix-core
// instruction, and it is what the tile hierarchy below feeds.
//
// The kernels compute C = alpha * op(A) * op(B) + beta * C (the general form
// of section 07's vendor call); each transpose pair is its own instantiation,
// built in its own translation unit (mfma_nn.hip, ...).
//
// Hierarchy
//  * work-group: BM x BN tile of C, WAVES_M x WAVES_N waves, K walked in
//    slabs of BK; slab t+1 is fetched into registers while slab t is
//    multiplied out of LDS, then written to the other of two LDS buffers
//    (one barrier per slab);
//  * wave: WM x WN = (BM / WAVES_M) x (BN / WAVES_N) tile, held as
//    (WM / 32) x (WN / 32) accumulator blocks of 32 x 32 (16 VGPRs each);
//  * instruction: v_mfma_f32_32x32x2_f32, C[32x32] += A[32x2] * B[2x32].
//    Lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32]; accumulator
//    register r of lane l is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
//
// Operands. The instruction treats its two operands alike: lane l gives the
// operand's free index (row of A, column of B) l % 32 and its k index l / 32.
// So each operand tile is described the same way (struct Operand), by how it
// is stored: with k contiguous (A as given, or B transposed: "KC") or with the
// free index contiguous (B as given, or A transposed: "FC"). The tile keeps
// its storage order in LDS, so global memory is copied to LDS in 16-byte
// chunks in every case, and the K order inside a slab (free: any order of the
// terms gives the sum) is chosen to make every LDS read wide:
//  * within a group of 8 consecutive k, MFMA step s (0..3) gives lane half h
//    the k index 4h + s. From a KC tile a lane then reads the four values
//    X[f][4h .. 4h+3] for the four steps with one 16-byte read;
//  * from an FC tile the 32 lanes of one block are interleaved TI-ways: block
//    t of a group covers free indices TI*c + t, c = 0..31, so lane c reads the
//    TI adjacent values X[k][TI*c .. TI*c+TI-1] in one read and feeds element
//    t to block t. In the epilogue a lane then holds TI adjacent columns of C
//    (B as given) and stores them with one wide store.
// KC rows in LDS carry 4 words of padding so the 32 rows read by a half-wave
// at the same k fall in distinct banks; FC rows are read as contiguous spans
// and are not padded.
//
// Ragged shapes: one launch covers C with tiles of one shape; the tiles that
// cross its bottom or right edge run the same loop with their reads clamped
// into the operands and their stores guarded (interior_tile), and a partial
// last slab of K reads zeros past K. Products whose row-contiguous operand
// is under 4 wide use general_tile, which guards every element instead.
#pragma once

#include <type_traits>

#include "gemm.hpp"
#include "tile_io.hpp"
#include "wsplit.hpp"

namespace sgemm_impl {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
// Native short vectors: copies of them stay in registers (copies of the HIP
// float4 struct through pointers become memcpy and can end up in scratch).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int N>
struct VecT;
template <>
struct VecT<1> {
    using T = float;
};
template <>
struct VecT<2> {
    using T = f32x2;
};
template <>
struct VecT<4> {
    using T = f32x4;
};

[[maybe_unused]] __device__ __forceinline__ float elem(float v, int) { return v; }
template <class V>
__device__ __forceinline__ float elem(V v, int t)
{
    return v[t];
}

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int REG_SETS_ = 1>
struct MfmaConfig {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
    // Register sets that stage slabs on their way global -> LDS: with one,
    // a slab's loads are issued one slab before it is stored to LDS; with two,
    // two slabs before.
    static constexpr int kRegSets = REG_SETS_;
    static_assert(kRegSets == 1 || kRegSets == 2, "one or two staging register sets");
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int kGroupM = SGEMM_MFMA_GROUP_M;
    // Waves per SIMD the register allocation aims at: one when a wave's
    // accumulators alone fill the 256 AGPRs, more as they shrink.
    static constexpr int kAccRegs = (WM / 32) * (WN / 32) * 16;
    // A second staging set needs more than the 128 registers of four waves
    // per SIMD, so such a tile runs two (one eight-wave work-group per CU).
    static constexpr int kWavesPerEU = kAccRegs >= 256 ? 1 : (kAccRegs >= 64 || REG_SETS_ == 2) ? 2 : 4;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK % 8 == 0, "slab depth must be whole groups of 8");
};

// One operand's share of a work-group tile: F free indices (rows of op(A)'s
// tile, or columns of op(B)'s) by BK values of k, of which each wave
// multiplies W free indices, copied by NT work-items. KC: stored with k
// contiguous; otherwise with the free index contiguous. In LDS (one stage):
//   KC: F rows of BK values, padded by 4 words: lds[f * (BK + 4) + k];
//   FC: BK rows of F values:                    lds[k * F + f].
// A "stored row" is a row of the operand as it lies in memory: a free index
// (KC) or a k (FC).
template <int F, int W, int BK, int NT, bool KC_>
struct Operand {
    static constexpr bool KC = KC_;
    static constexpr int NB = W / 32;                          // MFMA blocks per wave
    static constexpr int TI = KC ? 1 : W % 128 == 0 ? 4 : W % 64 == 0 ? 2 : 1;  // blocks fed by one LDS read
    static constexpr int NJ = NB / TI;                         // LDS reads per step (FC)
    static constexpr int kPitch = KC ? BK + 4 : F;             // LDS row pitch, floats
    static constexpr int kFloats = KC ? F * (BK + 4) : BK * F;
    static constexpr int kRows = KC ? F : BK;                  // stored rows in a tile
    static constexpr int kRowLen = KC ? BK : F;                // stored row length in a tile
    static constexpr int kRowChunks = kRowLen / 4;             // 16-byte chunks per stored row
    static constexpr int kChunks = F * BK / 4 / NT;            // chunks per work-item per slab
    static constexpr int kThreadsPerSlab = NT;                 // work-items sharing a slab's chunks
    // With NT a multiple of the chunks per stored row, a work-item's chunks lie
    // kRowStep stored rows apart in one column; otherwise each has its own row
    // and column (kEven false).
    static constexpr bool kEven = NT % kRowChunks == 0;
    static constexpr int kRowStep = NT / kRowChunks;           // stored rows between them (kEven)
    static constexpr int kReads = KC ? NB : 4 * NJ;            // LDS reads per group of 8 k
    using V = typename VecT<TI>::T;
    static_assert(TI == 1 || TI == 2 || TI == 4, "interleave must be 1, 2 or 4");
    static_assert(NB == NJ * TI, "wave tile must split into interleaved groups");
    static_assert(kChunks * 4 * NT == F * BK, "tile must split evenly over the work-items");

    // Free index, within the wave's W, of lane column c (0..31) of block b.
    __device__ static constexpr int free_index(int b, int c)
    {
        return KC ? b * 32 + c : (b / TI) * (32 * TI) + c * TI + b % TI;
    }

    // Operand values of one group of 8 k: element (b, s) feeds block b at
    // MFMA step s.
    struct Frag {
        f32x4 kc[KC ? NB : 1];
        V fc[4][KC ? 1 : NJ];
        __device__ float get(int b, int s) const
        {
            if constexpr (KC)
                return kc[b][s];
            else
                return elem(fc[s][b / TI], b % TI);
        }
    };

    // Fragments of group g of the stage at `lds` for the wave whose free
    // indices start at w0 (lane column l32, lane half h).
    __device__ static void read(Frag &fr, const float *lds, int w0, int g, int l32, int h)
    {
        if constexpr (KC) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
                fr.kc[b] = *reinterpret_cast<const f32x4 *>(&lds[(w0 + b * 32 + l32) * kPitch + 8 * g + 4 * h]);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    fr.fc[s][j] =
                        *reinterpret_cast<const V *>(&lds[(8 * g + 4 * h + s) * F + w0 + j * 32 * TI + l32 * TI]);
        }
    }

    // Chunk c of a slab: stored row and column inside the tile, and its LDS
    // offset.
    __device__ static constexpr int chunk_row(int c) { return c / kRowChunks; }
    __device__ static constexpr int chunk_col(int c) { return (c % kRowChunks) * 4; }
    __device__ static constexpr int chunk_lds(int c) { return chunk_row(c) * kPitch + chunk_col(c); }

    // Global (stored row, column) of tile element (r, c) of the slab at k0,
    // for the tile whose free indices start at f0.
    __device__ static std::int64_t global_row(std::int64_t f0, int k0, int r) { return KC ? f0 + r : k0 + r; }
    __device__ static int global_col(std::int64_t f0, int k0, int c) { return KC ? k0 + c : int(f0) + c; }
};

// Operand tiles of one configuration and transpose pair: A is KC unless
// transposed, B is KC only when transposed.
template <class Cfg, bool TA, bool TB>
struct Tiles {
    using OpA = Operand<Cfg::BM, Cfg::WM, Cfg::BK, Cfg::kThreads, !TA>;
    using OpB = Operand<Cfg::BN, Cfg::WN, Cfg::BK, Cfg::kThreads, TB>;
    static constexpr int kLdsFloats = 2 * (OpA::kFloats + OpB::kFloats);  // two stages
};

// Memory a stored operand is read from: base, leading dimension, and the
// extent of its free index (M for A, N for B).
struct OperandRef {
    const float *X;
    std::int64_t ld;
    std::int64_t free_extent;
};

// How OperandSource::place rotates an FC chunk at the edge (see there).
enum class Rotate { kSelect, kSelectPinned, kBranch };

// Where one work-item's chunks of an operand tile come from, for the fast
// tile body: chunk q of every slab starts at chunk(q) + slab offset. With
// EDGE, addresses are clamped into the operand (see interior_tile) and
// place() rotates an FC chunk read from a shifted address back into place.
// When the work-items' chunks advance evenly (Op::kEven) one offset and one
// shift serve every chunk; otherwise each chunk keeps its own.
template <class Op, bool EDGE>
struct OperandSource {
    static constexpr bool kPerChunk = (EDGE && Op::KC) || !Op::kEven;
    static constexpr int kOffs = kPerChunk ? Op::kChunks : 1;
    static constexpr int kShifts = (EDGE && !Op::KC && !Op::kEven) ? Op::kChunks : 1;
    const float *base;
    std::int64_t ld;
    std::int64_t off[kOffs];  // per-chunk offsets where needed
    int shift[kShifts];       // FC: elements the read was moved left

    __device__ OperandSource(const float *X, std::int64_t ld_, std::int64_t f0, std::int64_t extent, int tid)
        : base(X), ld(ld_)
    {
#pragma unroll
        for (int q = 0; q < kOffs; ++q) {
            const int c = tid + q * Op::kThreadsPerSlab;
            const int r0 = Op::chunk_row(c), c0 = Op::chunk_col(c);
            if constexpr (Op::KC) {  // stored rows are free indices, columns are k
                std::int64_t f = f0 + r0;
                if constexpr (EDGE) f = f < extent ? f : extent - 1;
                off[q] = f * ld + c0;
            } else {  // stored rows are k, columns are free indices
                std::int64_t f = f0 + c0;
                if constexpr (EDGE) {
                    const std::int64_t last = extent - 4;  // extent >= 4
                    const std::int64_t fr = f < last ? f : last;
                    const std::int64_t d = f - fr;
                    if (q < kShifts) shift[q] = int(d < 3 ? d : 3);
                    f = fr;
                }
                off[q] = std::int64_t(r0) * ld + f;
            }
        }
        if constexpr (!EDGE || Op::KC) shift[0] = 0;
    }
    __device__ const float *chunk(int q) const
    {
        if constexpr (kPerChunk)
            return base + off[q];
        else
            return base + off[0] + std::int64_t(q) * Op::kRowStep * ld;
    }
    // Element e of chunk q is element e + shift of what was read (the
    // elements past the operand's edge keep junk). Three forms, chosen per
    // loop by measurement:
    //  * kSelect: two steps of one independent select each (by 1, then by
    //    2), straight-line code. A chain of compares of the shift against 0,
    //    1 and 2 becomes a switch, compiled to divergent branches that split
    //    a slab loop's interleaved schedule (the 256 x 256 tile's edge tiles
    //    ran 4-5% slower with it);
    //  * kSelectPinned: the same behind an empty asm that ties the rotation
    //    to the point of the code where the chunk is stored. Free to move in
    //    a loop with two staging register sets, the selects were computed for
    //    both sets at the top of the loop, which then waited for the newest
    //    loads in flight as well;
    //  * kBranch: the compare chain; its branches skip the rotation in waves
    //    with no chunk at the edge, which pays in the short slabs of the
    //    two-set 64 x 64 tile.
    template <Rotate R>
    __device__ f32x4 place(f32x4 v, int q) const
    {
        if constexpr (EDGE && !Op::KC) {
            const int s = shift[kShifts > 1 ? q : 0];
            f32x4 r;
            if constexpr (R == Rotate::kBranch) {
                r[0] = s == 0 ? v[0] : s == 1 ? v[1] : s == 2 ? v[2] : v[3];
                r[1] = s == 0 ? v[1] : s == 1 ? v[2] : v[3];
                r[2] = s == 0 ? v[2] : v[3];
            } else {
                if constexpr (R == Rotate::kSelectPinned) asm volatile("" : "+v"(v));
                const bool b0 = (s & 1) != 0, b1 = (s & 2) != 0;
                const float t0 = b0 ? v[1] : v[0], t1 = b0 ? v[2] : v[1], t2 = b0 ? v[3] : v[2];
                r[0] = b1 ? t2 : t0;
                r[1] = b1 ? v[3] : t1;
                r[2] = b1 ? v[3] : t2;
            }
            r[3] = v[3];
            return r;
        } else {
            return v;
        }
    }
};

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100, kSchedDsWrite = 0x200;

// f(std::integral_constant<int, I>{}) for I = B .. E-1, unrolled.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Zero accumulators.
template <int NA, int NB>
__device__ __forceinline__ void clear(floatx16 (&acc)[NA][NB])
{
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = floatx16{};
}

// The four MFMA steps of one group of 8 k.
template <class OpA, class OpB>
__device__ __forceinline__ void mfma_group(floatx16 (&acc)[OpA::NB][OpB::NB], const typename OpA::Frag &fa,
                                           const typename OpB::Frag &fb)
{
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int a = 0; a < OpA::NB; ++a)
#pragma unroll
            for (int b = 0; b < OpB::NB; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.get(a, s), fb.get(b, s), acc[a][b], 0, 0, 0);
}

// Epilogue: C <- alpha * acc + beta * C for the wave's blocks. Register r of
// block (a, b) is row OpA::free_index(a, 8(r/4) + 4h + r%4) and column
// OpB::free_index(b, l32) of the wave tile; the TI blocks of one FC group of
// B give a lane TI adjacent columns, updated with one access.
//
// With beta != 0 the old values of C are read a block (16 rows of TI
// columns) at a time, all before any of them is written.
template <class OpA, class OpB>
__device__ __forceinline__ void write_tile(const Problem &p, const floatx16 (&acc)[OpA::NB][OpB::NB],
                                           std::int64_t r0, int c0, int l32, int h, bool inside)
{
    constexpr int TB = OpB::TI;
    if (p.beta != 0.0f) {
#pragma unroll
        for (int a = 0; a < OpA::NB; ++a)
#pragma unroll
            for (int j = 0; j < OpB::NJ; ++j) {
                const int col = c0 + j * 32 * TB + l32 * TB;
                float old[16][TB];
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    read_c<TB>(p.C, p.ldc, r0 + OpA::free_index(a, 8 * (r / 4) + 4 * h + (r % 4)), col, p.M, p.N,
                               inside, old[r]);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float v[TB];
#pragma unroll
                    for (int t = 0; t < TB; ++t) v[t] = acc[a][j * TB + t][r];
                    write_c<TB>(p.C, p.ldc, r0 + OpA::free_index(a, 8 * (r / 4) + 4 * h + (r % 4)), col, p.M, p.N,
                                v, old[r], inside, p.alpha, p.beta);
                }
            }
        return;
    }
#pragma unroll
    for (int a = 0; a < OpA::NB; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const std::int64_t row = r0 + OpA::free_index(a, 8 * (r / 4) + 4 * h + (r % 4));
#pragma unroll
            for (int j = 0; j < OpB::NJ; ++j) {
                const int col = c0 + j * 32 * TB + l32 * TB;
                float v[TB];
#pragma unroll
                for (int t = 0; t < TB; ++t) v[t] = acc[a][j * TB + t][r];
                update_n<TB>(p.C, p.ldc, row, col, p.M, p.N, v, inside, p.alpha, p.beta);
            }
        }
}

// One BM x BN tile (tm, tn) of the product p, with guards on every edge;
// `lds` holds Tiles<Cfg, TA, TB>::kLdsFloats floats.
template <class Cfg, bool TA, bool TB, bool VEC>
__device__ __forceinline__ void general_tile(const Problem &p, int tm, int tn, float *lds)
{
    using T = Tiles<Cfg, TA, TB>;
    using OpA = typename T::OpA;
    using OpB = typename T::OpB;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::kThreads;
    constexpr int G = BK / 8;  // groups of 8 k per slab

    float(*As)[OpA::kFloats] = reinterpret_cast<float(*)[OpA::kFloats]>(lds);
    float(*Bs)[OpB::kFloats] = reinterpret_cast<float(*)[OpB::kFloats]>(lds + 2 * OpA::kFloats);

    const std::int64_t m0 = std::int64_t(tm) * BM;
    const int n0 = tn * BN;
    const OperandRef ra_{p.A, p.lda, p.M}, rb_{p.B, p.ldb, p.N};

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

    floatx16 acc[OpA::NB][OpB::NB];
    clear(acc);

    // Global -> register staging of one slab: chunk c of an operand tile is
    // stored row chunk_row(c), columns chunk_col(c) .. +3.
    float4 ra[OpA::kChunks], rb[OpB::kChunks];
    auto fetch_op = [&](auto op, const OperandRef &x, std::int64_t f0, int k0, float4 *r, auto guarded) {
        using Op = decltype(op);
#pragma unroll
        for (int q = 0; q < Op::kChunks; ++q) {
            const int c = tid + q * NT;
            const std::int64_t row = Op::global_row(f0, k0, Op::chunk_row(c));
            const int col = Op::global_col(f0, k0, Op::chunk_col(c));
            if constexpr (decltype(guarded)::value) {
                const std::int64_t rows = Op::KC ? x.free_extent : p.K;
                const int cols = Op::KC ? p.K : int(x.free_extent);
                r[q] = load4_clamped(x.X, x.ld, row, col, rows, cols);
            } else {
                r[q] = load4_inside<VEC>(x.X, x.ld, row, col);
            }
        }
    };
    auto stash_op = [&](auto op, const OperandRef &x, std::int64_t f0, int k0, float4 *r, float *dst,
                        auto guarded) {
        using Op = decltype(op);
#pragma unroll
        for (int q = 0; q < Op::kChunks; ++q) {
            const int c = tid + q * NT;
            if constexpr (decltype(guarded)::value) {
                const std::int64_t rows = Op::KC ? x.free_extent : p.K;
                const int cols = Op::KC ? p.K : int(x.free_extent);
                zero_outside(r[q], Op::global_row(f0, k0, Op::chunk_row(c)), Op::global_col(f0, k0, Op::chunk_col(c)),
                             rows, cols);
            }
            *reinterpret_cast<float4 *>(&dst[Op::chunk_lds(c)]) = r[q];
        }
    };
    auto fetch = [&](int slab, auto guarded) {
        fetch_op(OpA{}, ra_, m0, slab * BK, ra, guarded);
        fetch_op(OpB{}, rb_, n0, slab * BK, rb, guarded);
    };
    auto stash = [&](int buf, int slab, auto guarded) {
        stash_op(OpA{}, ra_, m0, slab * BK, ra, As[buf], guarded);
        stash_op(OpB{}, rb_, n0, slab * BK, rb, Bs[buf], guarded);
    };

    // Operand fragments of one group of 8 k, double-buffered in registers so
    // the reads of group g+1 are in flight while group g's MFMAs issue.
    typename OpA::Frag fa[2];
    typename OpB::Frag fb[2];
    auto read_frags = [&](int buf, int g, int slot) {
        OpA::read(fa[slot], As[buf], wm0, g, l32, h);
        OpB::read(fb[slot], Bs[buf], wn0, g, l32, h);
    };
    auto mfmas = [&](int slot) { mfma_group<OpA, OpB>(acc, fa[slot], fb[slot]); };
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

    write_tile<OpA, OpB>(p, acc, m0 + wm0, n0 + wn0, l32, h, interior);
}

// The fast tile body. Rows need only the 4-byte alignment of any float:
// global memory moves in 16-byte accesses that gfx950 performs unaligned. The
// partial last slab (K not a multiple of BK) is loaded once, with guards,
// after the loop. Same operand order and LDS layout as general_tile; the slab
// loop is arranged for few waves per SIMD:
//  * each steady-state slab is one straight-line block whose LDS stores,
//    global loads and fragment reads are spread one per MFMA (a burst of
//    memory instructions would hold back the next MFMA, as a wave issues in
//    order);
//  * the barrier sits before the last group of k of the slab, so the first
//    fragments of the next slab load while that group is multiplied.
//
// EDGE tiles (crossing the bottom or right edge of C) run the same loop with
// no guard in it: every address is kept inside the operand instead.
//  * A chunk whose free index (a KC row) lies past the operand's extent is
//    read from the last valid row: its values only reach rows or columns of
//    C that are never stored.
//  * An FC chunk (4 consecutive free indices) that crosses the edge is read
//    from the last 4 valid elements of its row, and rotated in registers
//    when it is stored to LDS so each valid element lands in its place; a
//    chunk wholly past the edge is read from there too (its values are never
//    used). This needs the FC free extent >= 4.
//  * Only k must read as zero outside [0, K), and full slabs never leave it;
//    the partial slab is loaded element by element as before. Stores are
//    guarded.
// interior_tile computes the BM x BN tile (tm, tn) of the product p; `lds`
// holds Tiles<Cfg, TA, TB>::kLdsFloats floats. With RANGE it sums only the
// slabs [rg.s_begin, rg.s_end) of K (slab n_full being the partial one, if K
// is not a multiple of BK) and, when rg.ws is set, stores the unscaled sum
// row-major into rg.ws (BM x BN floats) instead of updating C.
struct TileRange {
    int s_begin, s_end;
    float *ws;
};

template <class Cfg, bool TA, bool TB, bool EDGE, bool RANGE = false>
__device__ __forceinline__ void interior_tile(const Problem &p, int tm, int tn, float *lds, const TileRange &rg = {})
{
    using T = Tiles<Cfg, TA, TB>;
    using OpA = typename T::OpA;
    using OpB = typename T::OpB;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::kThreads;
    constexpr int G = BK / 8;
    constexpr int CA = OpA::kChunks, CB = OpB::kChunks;

    float(*As)[OpA::kFloats] = reinterpret_cast<float(*)[OpA::kFloats]>(lds);
    float(*Bs)[OpB::kFloats] = reinterpret_cast<float(*)[OpB::kFloats]>(lds + 2 * OpA::kFloats);

    const std::int64_t m0 = std::int64_t(tm) * BM;
    const int n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int l32 = lane % 32, h = lane / 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wm0 = (wave / Cfg::WAVES_N) * Cfg::WM;
    const int wn0 = (wave % Cfg::WAVES_N) * Cfg::WN;
    const int n_full = p.K / BK;
    const int s_first = RANGE ? rg.s_begin : 0;                                 // first full slab
    const int s_stop = RANGE ? (rg.s_end < n_full ? rg.s_end : n_full) : n_full;  // past the last full slab
    const bool tail = n_full * BK < p.K && (!RANGE || rg.s_end > n_full);         // the partial slab

    floatx16 acc[OpA::NB][OpB::NB];
    clear(acc);

    // This work-item's chunks: chunk q of an operand is stored row
    // chunk_row(q*NT + tid) of the slab, kRowStep stored rows after chunk
    // q-1, always in the same column. A slab further along K is BK columns
    // (KC) or BK rows (FC) on.
    const OperandSource<OpA, EDGE> srca(p.A, p.lda, m0, p.M, tid);
    const OperandSource<OpB, EDGE> srcb(p.B, p.ldb, n0, p.N, tid);
    const std::int64_t slab_a = OpA::KC ? BK : BK * p.lda, slab_b = OpB::KC ? BK : BK * p.ldb;

    // Slab s is staged in register set s % RS; `set` is always a constant
    // after unrolling, so the sets stay in fixed registers.
    constexpr int RS = Cfg::kRegSets;
    constexpr Rotate kRot = RS > 1 ? Rotate::kSelectPinned : Rotate::kSelect;
    f32x4 ra[RS][CA], rb[RS][CB];
    auto fetch = [&](int slab, int set) {  // slab counted from s_first
        const std::int64_t ka = (s_first + slab) * slab_a, kb = (s_first + slab) * slab_b;
#pragma unroll
        for (int q = 0; q < CA; ++q)
            ra[set][q] = load16u(srca.chunk(q) + ka);
#pragma unroll
        for (int q = 0; q < CB; ++q)
            rb[set][q] = load16u(srcb.chunk(q) + kb);
    };
    auto stash = [&](int buf, int set) {
#pragma unroll
        for (int q = 0; q < CA; ++q)
            *reinterpret_cast<f32x4 *>(&As[buf][OpA::chunk_lds(q * NT + tid)]) =
                srca.template place<kRot>(ra[set][q], q);
#pragma unroll
        for (int q = 0; q < CB; ++q)
            *reinterpret_cast<f32x4 *>(&Bs[buf][OpB::chunk_lds(q * NT + tid)]) =
                srcb.template place<kRot>(rb[set][q], q);
    };

    typename OpA::Frag fa[2];
    typename OpB::Frag fb[2];
    auto read_frags = [&](int buf, int g, int slot) {
        OpA::read(fa[slot], As[buf], wm0, g, l32, h);
        OpB::read(fb[slot], Bs[buf], wn0, g, l32, h);
    };
    auto mfmas = [&](int slot) { mfma_group<OpA, OpB>(acc, fa[slot], fb[slot]); };
    auto multiply = [&](int buf) {
        read_frags(buf, 0, 0);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g + 1 < G) read_frags(buf, g + 1, (g + 1) & 1);
            mfmas(g & 1);
        }
    };

    static_assert(G % 2 == 0, "the pipelined loop needs an even number of k-groups per slab");
    constexpr int NR = OpA::kReads + OpB::kReads;  // fragment reads per group
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

    const int n = s_stop - s_first;
    if (n > 0) {
        fetch(0, 0);
        stash(0, 0);
        // The next slabs' loads are issued whether or not the slabs exist
        // (slab 0 again in their place, never stored): with the loads under
        // a branch, the compiler's count of loads in flight at the loop's
        // head is the one of the path without them, and it then waits for
        // every load before the last LDS store of each pass, the newer
        // set's included.
        fetch(n > 1 ? 1 : 0, RS - 1);
        if constexpr (RS == 2) fetch(n > 2 ? 2 : 0, 0);
        __syncthreads();
        read_frags(0, 0, 0);
        int t = 0;
        // Steady state, one straight-line block per slab t (LDS buffer cur):
        //   A: store slab t+1 (registers) to buffer cur^1, start loading slab
        //      t+1+RS into the registers just freed, read groups 1..G-1 of
        //      slab t while multiplying groups 0..G-2;
        //   barrier: slab t+1 is complete in LDS, and every wave has finished
        //      reading buffer cur^1's previous contents (slab t-1, before the
        //      previous barrier);
        //   B: read group 0 of slab t+1 while multiplying group G-1 of slab t.
        if constexpr (RS == 1) {
            for (; t + 2 < n; ++t) {
                const int cur = t & 1;
                stash(cur ^ 1, 0);
                fetch(t + 2, 0);
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
        } else {
            // Two slabs per iteration, so that each names its register set
            // as a constant (slab t+1 is in set (t+1) & 1, and t is even).
            static_assert(CA + CB < 16, "the wait count below fits its field");
            auto steady = [&](int t, auto set) {
                const int cur = t & 1;
                // Loads complete in order, so at most CA + CB outstanding
                // (the other set's) means this set's have landed. The
                // compiler's own count would also wait for the other set.
                __builtin_amdgcn_s_waitcnt(0x0F70 | (CA + CB));  // vmcnt(CA+CB), expcnt/lgkmcnt: no wait
                stash(cur ^ 1, decltype(set)::value);
                fetch(t + 3, decltype(set)::value);
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
            };
            for (; t + 4 < n; t += 2) {
                steady(t, std::integral_constant<int, 1>{});
                steady(t + 1, std::integral_constant<int, 0>{});
            }
            if (t + 3 < n) steady(t++, std::integral_constant<int, 1>{});
        }
        // Last slabs: no more loads.
        for (; t < n; ++t) {
            const int cur = t & 1;
            if (t + 1 < n) {
                if (RS == 2 && ((t + 1) & 1) == 1)
                    stash(cur ^ 1, RS - 1);
                else
                    stash(cur ^ 1, 0);
            }
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
    if (tail) {
        // Partial last slab: k >= K reads as zero. Written straight to LDS one
        // element at a time; this runs once.
        const int k0 = n_full * BK;
        // Free indices past the operand's extent are clamped into it (their
        // values are never used), as in the loop.
        auto partial = [&](auto op, const float *X, std::int64_t ld, std::int64_t f0, std::int64_t extent,
                           float *dst) {
            using Op = decltype(op);
            // Batches of this work-item's loads first, then their LDS stores,
            // so that the loads of a batch are in flight together (the split
            // schedule's tile body, short of registers, takes one at a time).
            constexpr int kPer = Op::kRows * Op::kRowLen / NT;
            static_assert(kPer * NT == Op::kRows * Op::kRowLen, "whole elements per work-item");
            constexpr int kBatch = RANGE ? 1 : kPer;
            static_assert(kPer % kBatch == 0, "whole batches");
#pragma unroll 1
            for (int i0 = 0; i0 < kPer; i0 += kBatch) {
                float v[kBatch];
#pragma unroll
                for (int i = 0; i < kBatch; ++i) {
                    const int e = tid + (i0 + i) * NT;
                    const int r = e / Op::kRowLen, c = e % Op::kRowLen;
                    const int k = Op::KC ? c : r;
                    const std::int64_t f = f0 + (Op::KC ? r : c);
                    const std::int64_t fc = f < extent ? f : extent - 1;
                    const std::int64_t at = Op::KC ? fc * ld + k0 + k : std::int64_t(k0 + k) * ld + fc;
                    v[i] = k0 + k < p.K ? X[at] : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < kBatch; ++i) {
                    const int e = tid + (i0 + i) * NT;
                    dst[(e / Op::kRowLen) * Op::kPitch + e % Op::kRowLen] = v[i];
                }
            }
        };
        partial(OpA{}, p.A, p.lda, m0, p.M, As[0]);
        partial(OpB{}, p.B, p.ldb, n0, p.N, Bs[0]);
        __syncthreads();
        multiply(0);
    }

    if (RANGE && rg.ws != nullptr) {
        Problem q = p;  // the partial tile, unscaled, all of it
        q.C = rg.ws;
        q.ldc = BN;
        q.alpha = 1.0f;
        q.beta = 0.0f;
        write_tile<OpA, OpB>(q, acc, wm0, wn0, l32, h, true);
    } else {
        write_tile<OpA, OpB>(p, acc, m0 + wm0, n0 + wn0, l32, h, !EDGE);
    }
}

// A tile computed by KGROUPS sets of WAVES_M x WAVES_N waves, set g taking
// its own share (BK / 8 / KGROUPS groups of 8 k) of every slab; the sets'
// partial tiles are summed at the end. For products with one small tile per
// compute unit, this puts KGROUPS waves on each SIMD instead of one.
// Slabs are staged global -> registers -> LDS through REG_SETS register sets:
// slab t+1+REG_SETS is requested while slab t is multiplied.
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int KGROUPS_, int REG_SETS_ = 1>
struct KSplitConfig {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, KGROUPS = KGROUPS_;
    static constexpr int kRegSets = REG_SETS_;
    static_assert(kRegSets >= 1 && kRegSets <= 4, "one to four staging register sets");
    static constexpr int kThreads = 64 * WAVES_M * WAVES_N * KGROUPS;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int kGroupM = SGEMM_MFMA_GROUP_M;
    static constexpr int kAccRegs = (WM / 32) * (WN / 32) * 16;
    static constexpr int kWavesPerEU = kAccRegs >= 128 ? 2 : 4;
    static constexpr int kGroupsPerWave = BK / 8 / KGROUPS;
    static_assert(KGROUPS == 2, "the two partial tiles are summed pairwise");
    static_assert(kGroupsPerWave >= 1 && kGroupsPerWave * 8 * KGROUPS == BK, "whole groups of 8 per set");
};

template <class Cfg, bool TA, bool TB, bool EDGE>
__device__ __forceinline__ void ksplit_tile(const Problem &p, int tm, int tn, float *lds)
{
    using T = Tiles<Cfg, TA, TB>;
    using OpA = typename T::OpA;
    using OpB = typename T::OpB;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::kThreads;
    constexpr int GW = Cfg::kGroupsPerWave;
    // The steady loop reads the next slab's first group into fragment slot 0
    // before it multiplies this slab's last group, so that group must sit in
    // slot 1: an even number of groups per wave.
    static_assert(GW % 2 == 0, "the pipelined loop needs an even number of k-groups per wave");
    constexpr int CA = OpA::kChunks, CB = OpB::kChunks;
    constexpr int NS = Cfg::WAVES_M * Cfg::WAVES_N;  // waves per set

    float(*As)[OpA::kFloats] = reinterpret_cast<float(*)[OpA::kFloats]>(lds);
    float(*Bs)[OpB::kFloats] = reinterpret_cast<float(*)[OpB::kFloats]>(lds + 2 * OpA::kFloats);

    const std::int64_t m0 = std::int64_t(tm) * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int l32 = lane % 32, h = lane / 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int set = wave / NS, sw = wave % NS;
    const int wm0 = (sw / Cfg::WAVES_N) * Cfg::WM;
    const int wn0 = (sw % Cfg::WAVES_N) * Cfg::WN;
    const int g0 = set * GW;
    const int n_full = p.K / BK;

    floatx16 acc[OpA::NB][OpB::NB];
    clear(acc);

    const OperandSource<OpA, EDGE> srca(p.A, p.lda, m0, p.M, tid);
    const OperandSource<OpB, EDGE> srcb(p.B, p.ldb, n0, p.N, tid);
    const std::int64_t slab_a = OpA::KC ? BK : BK * p.lda, slab_b = OpB::KC ? BK : BK * p.ldb;

    // Slab s is staged in register set s % RS; in the steady loop `set` is
    // a constant after unrolling, so the sets stay in fixed registers.
    constexpr int RS = Cfg::kRegSets;
    f32x4 ra[RS][CA], rb[RS][CB];
    auto fetch = [&](int slab, int set) {
        const std::int64_t ka = slab * slab_a, kb = slab * slab_b;
#pragma unroll
        for (int q = 0; q < CA; ++q)
            ra[set][q] = load16u(srca.chunk(q) + ka);
#pragma unroll
        for (int q = 0; q < CB; ++q)
            rb[set][q] = load16u(srcb.chunk(q) + kb);
    };
    auto stash = [&](int buf, int set) {
#pragma unroll
        for (int q = 0; q < CA; ++q)
            *reinterpret_cast<f32x4 *>(&As[buf][OpA::chunk_lds(q * NT + tid)]) =
                srca.template place<Rotate::kBranch>(ra[set][q], q);
#pragma unroll
        for (int q = 0; q < CB; ++q)
            *reinterpret_cast<f32x4 *>(&Bs[buf][OpB::chunk_lds(q * NT + tid)]) =
                srcb.template place<Rotate::kBranch>(rb[set][q], q);
    };
    // The same with a set known only at run time (the loop's last slabs).
    auto stash_any = [&](int buf, int set) {
        static_for<0, RS>([&](auto i) {
            if (set == decltype(i)::value) stash(buf, decltype(i)::value);
        });
    };
    typename OpA::Frag fa[2];
    typename OpB::Frag fb[2];
    auto read_frags = [&](int buf, int g, int slot) {
        OpA::read(fa[slot], As[buf], wm0, g, l32, h);
        OpB::read(fb[slot], Bs[buf], wn0, g, l32, h);
    };
    auto mfmas = [&](int slot) { mfma_group<OpA, OpB>(acc, fa[slot], fb[slot]); };
    // This set's groups of one buffer whose first group is already read.
    auto multiply_mine = [&](int buf) {
#pragma unroll
        for (int gg = 0; gg < GW; ++gg) {
            if (gg + 1 < GW) read_frags(buf, g0 + gg + 1, (gg + 1) & 1);
            mfmas(gg & 1);
        }
    };
    // Interleave hints as in interior_tile: one memory instruction after
    // each MFMA, so the slab's stores and loads do not issue as one burst
    // that the next MFMA waits behind.
    constexpr int NR = OpA::kReads + OpB::kReads;  // fragment reads per group
    auto interleave_a = [&] {
#pragma unroll
        for (int i = 0; i < (GW - 1) * NR; ++i) {
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
        fetch(0, 0);
        stash(0, 0);
        // Under a branch, unlike interior_tile's: issued unconditionally,
        // these loads made the tile 1.4% slower at 1024 x 1024 x 4096.
#pragma unroll
        for (int s = 1; s <= RS; ++s)
            if (n > s) fetch(s, s % RS);
        __syncthreads();
        read_frags(0, g0, 0);
        int t = 0;
        // Steady state, one straight-line block per slab t (LDS buffer cur).
        // With the store and the load under a branch, the compiler cannot
        // count the LDS operations in flight and waits for all of them before
        // each slab's first MFMA; straight-line code waits for the fragments
        // only (+2-5% on products of one 64x64 tile per compute unit).
        //   store slab t+1 (register set (t+1) % RS) to buffer cur^1, start
        //   loading slab t+1+RS into that set, multiply this set's groups of
        //   slab t but the last;
        //   barrier: slab t+1 is complete in LDS, and every wave has finished
        //   reading buffer cur^1's previous contents (slab t-1);
        //   read this set's first group of slab t+1 and multiply the last
        //   group of slab t (the scheduler may lift those MFMAs above the
        //   barrier; pinning them below it with sched_barrier measured 4-8%
        //   slower).
        auto steady = [&](int t, auto setc) {
            constexpr int set = decltype(setc)::value;
            const int cur = t & 1;
            if constexpr (RS > 1) {
                // Loads complete in order: with at most the newer sets' loads
                // outstanding, this set's have landed. The compiler's own
                // count would also wait for the newer sets.
                static_assert((RS - 1) * (CA + CB) < 16, "the wait count fits its field");
                __builtin_amdgcn_s_waitcnt(0x0F70 | ((RS - 1) * (CA + CB)));  // vmcnt only
            }
            stash(cur ^ 1, set);
            fetch(t + 1 + RS, set);
#pragma unroll
            for (int gg = 0; gg + 1 < GW; ++gg) {
                read_frags(cur, g0 + gg + 1, (gg + 1) & 1);
                mfmas(gg & 1);
            }
            interleave_a();
            __syncthreads();
            read_frags(cur ^ 1, g0, 0);
            mfmas((GW - 1) & 1);
            interleave_b();
        };
        // RS slabs per pass, so that slab t+1's set, (t+1) % RS, is a
        // constant in each (t is a multiple of RS at the top of a pass).
        for (; t + 2 * RS < n; t += RS)
            static_for<0, RS>([&](auto i) {
                steady(t + decltype(i)::value, std::integral_constant<int, (decltype(i)::value + 1) % RS>{});
            });
        static_for<0, RS - 1>([&](auto i) {
            if (t + RS + 1 < n) steady(t++, std::integral_constant<int, (decltype(i)::value + 1) % RS>{});
        });
        // Last RS + 1 slabs: no more loads.
        for (; t < n; ++t) {
            const int cur = t & 1;
            if (t + 1 < n) stash_any(cur ^ 1, (t + 1) % RS);
            multiply_mine(cur);
            __syncthreads();
            if (t + 1 < n) read_frags(cur ^ 1, g0, 0);
        }
    }
    if (n_full * BK < p.K) {
        const int k0 = n_full * BK;
        auto partial = [&](auto op, const float *X, std::int64_t ld, std::int64_t f0, std::int64_t extent,
                           float *dst) {
            using Op = decltype(op);
            // All of this work-item's loads first, then the LDS stores, so
            // that the loads are in flight together.
            constexpr int kPer = Op::kRows * Op::kRowLen / NT;
            static_assert(kPer * NT == Op::kRows * Op::kRowLen, "whole elements per work-item");
            float v[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int e = tid + i * NT;
                const int r = e / Op::kRowLen, c = e % Op::kRowLen;
                const int k = Op::KC ? c : r;
                const std::int64_t f = f0 + (Op::KC ? r : c);
                const std::int64_t fc = f < extent ? f : extent - 1;
                const std::int64_t at = Op::KC ? fc * ld + k0 + k : std::int64_t(k0 + k) * ld + fc;
                v[i] = k0 + k < p.K ? X[at] : 0.0f;
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
        read_frags(0, g0, 0);
        multiply_mine(0);
        __syncthreads();
    }

    // Set 1's partial tile through LDS into set 0's: register r of lane l of
    // block (a, b) of spatial wave sw at red[((sw * NA + a) * NB + b) * 16 + r) * 64 + l].
    constexpr int NA = OpA::NB, NBb = OpB::NB;
    float *red = lds;
    if (set == 1) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int b = 0; b < NBb; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) red[(((sw * NA + a) * NBb + b) * 16 + r) * 64 + lane] = acc[a][b][r];
    }
    __syncthreads();
    if (set == 0) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int b = 0; b < NBb; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[a][b][r] += red[(((sw * NA + a) * NBb + b) * 16 + r) * 64 + lane];
        write_tile<OpA, OpB>(p, acc, m0 + wm0, n0 + wn0, l32, h, !EDGE);
    }
}

// Tile shapes (tiles.hpp).
using GeneralCfg = MfmaConfig<SGEMM_MFMA_TILE>;
using BigCfg = MfmaConfig<SGEMM_MFMA_BIG_TILE>;
using MidCfg = MfmaConfig<SGEMM_MFMA_MID_TILE, SGEMM_MFMA_MID_REG_SETS>;
// Four waves whose 64 accumulator registers a wave and two staging sets fit
// the budget of two waves per SIMD: two such work-groups per compute unit.
using MidDualCfg = MfmaConfig<SGEMM_MFMA_MID_DUAL_TILE, SGEMM_MFMA_MID_DUAL_REG_SETS>;
static_assert(MidDualCfg::kWavesPerEU * 4 == 2 * MidDualCfg::kThreads / 64, "two work-groups per compute unit");
// The split schedule's 128x128 pieces run two work-groups per compute unit
// too: the four-wave tile, with one staging set (two measured the same). They
// ran 4-6% faster than eight-wave pieces with one set (interleaved medians on
// MI355X, TFLOP/s: 1536^3 95.2 -> 100.6, 512 x 512 x 16384 103.2 -> 107.7,
// 768 x 768 x 8192 108.0 -> 112.5).
using MidSplitCfg = MfmaConfig<SGEMM_MFMA_MID_DUAL_TILE>;
using SmallCfg = MfmaConfig<SGEMM_MFMA_SMALL_TILE>;
using WideCfg = MfmaConfig<SGEMM_MFMA_WIDE_TILE, SGEMM_MFMA_WIDE_REG_SETS>;
using WideNCfg = MfmaConfig<SGEMM_MFMA_WIDEN_TILE, SGEMM_MFMA_WIDEN_REG_SETS>;
using KSplitCfg = KSplitConfig<SGEMM_MFMA_KSPLIT_TILE, SGEMM_MFMA_KSPLIT_REG_SETS>;
using KSplit32Cfg = KSplitConfig<SGEMM_MFMA_KSPLIT32_TILE, SGEMM_MFMA_KSPLIT_REG_SETS>;
using Ws64Cfg = WsConfig<SGEMM_MFMA_WSPLIT64>;
using Ws96Cfg = WsConfig<SGEMM_MFMA_WSPLIT96>;
using Ws128Cfg = WsConfig<SGEMM_MFMA_WSPLIT128>;

// Products too small for a single interior tile: general tiles only.
template <class Cfg, bool TA, bool TB, bool VEC>
__global__ __launch_bounds__(Cfg::kThreads) void mfma_kernel(Problem p, int tiles_m)
{
    __shared__ __attribute__((aligned(16))) float lds[Tiles<Cfg, TA, TB>::kLdsFloats];
    int tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, Cfg::kGroupM, tm, tn);
    general_tile<Cfg, TA, TB, VEC>(p, tm, tn, lds);
}

// One launch over all BM x BN tiles of the product: tiles that cross the
// bottom or right edge of C take the EDGE body of the same loop.
template <class Cfg, bool TA, bool TB>
__global__ __launch_bounds__(Cfg::kThreads)
__attribute__((amdgpu_waves_per_eu(Cfg::kWavesPerEU, Cfg::kWavesPerEU))) void mfma_tiles_kernel(Problem p, int tiles_m)
{
    __shared__ __attribute__((aligned(16))) float lds[Tiles<Cfg, TA, TB>::kLdsFloats];
    int tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, Cfg::kGroupM, tm, tn);
    const bool edge = std::int64_t(tm + 1) * Cfg::BM > p.M || std::int64_t(tn + 1) * Cfg::BN > p.N;
    if (edge)
        interior_tile<Cfg, TA, TB, true>(p, tm, tn, lds);
    else
        interior_tile<Cfg, TA, TB, false>(p, tm, tn, lds);
}

template <class Cfg, bool TA, bool TB>
__global__ __launch_bounds__(Cfg::kThreads)
__attribute__((amdgpu_waves_per_eu(Cfg::kWavesPerEU, Cfg::kWavesPerEU))) void mfma_ksplit_kernel(Problem p, int tiles_m)
{
    constexpr int kPipe = Tiles<Cfg, TA, TB>::kLdsFloats;
    constexpr int kRed = Cfg::WAVES_M * Cfg::WAVES_N * (Cfg::WM / 32) * (Cfg::WN / 32) * 16 * 64;
    __shared__ __attribute__((aligned(16))) float lds[kPipe > kRed ? kPipe : kRed];
    int tm, tn;
    tile_of_workgroup(blockIdx.x, gridDim.x, tiles_m, Cfg::kGroupM, tm, tn);
    const bool edge = std::int64_t(tm + 1) * Cfg::BM > p.M || std::int64_t(tn + 1) * Cfg::BN > p.N;
    if (edge)
        ksplit_tile<Cfg, TA, TB, true>(p, tm, tn, lds);
    else
        ksplit_tile<Cfg, TA, TB, false>(p, tm, tn, lds);
}

template <class Cfg, bool TA, bool TB>
hipError_t launch_ksplit(const Problem &p, hipStream_t stream)
{
    const void *kernel = reinterpret_cast<const void *>(&mfma_ksplit_kernel<Cfg, TA, TB>);
    return for_each_band<Cfg::BM, Cfg::BN>(p, [&](Problem q, int tiles_m, int tiles_n) {
        void *args[] = {&q, &tiles_m};
        return hipLaunchKernel(kernel, dim3(unsigned(tiles_m) * unsigned(tiles_n)), dim3(Cfg::kThreads), args, 0,
                               stream);
    });
}

template <class Cfg, bool TA, bool TB>
hipError_t launch_general(const Problem &p, hipStream_t stream)
{
    const void *kernel = rows_aligned16(p) ? reinterpret_cast<const void *>(&mfma_kernel<Cfg, TA, TB, true>)
                                           : reinterpret_cast<const void *>(&mfma_kernel<Cfg, TA, TB, false>);
    return for_each_band<Cfg::BM, Cfg::BN>(p, [&](Problem q, int tiles_m, int tiles_n) {
        void *args[] = {&q, &tiles_m};
        return hipLaunchKernel(kernel, dim3(unsigned(tiles_m) * unsigned(tiles_n)), dim3(Cfg::kThreads), args, 0,
                               stream);
    });
}

template <class Cfg, bool TA, bool TB>
hipError_t launch_tiles(const Problem &p, hipStream_t stream)
{
    const void *kernel = reinterpret_cast<const void *>(&mfma_tiles_kernel<Cfg, TA, TB>);
    return for_each_band<Cfg::BM, Cfg::BN>(p, [&](Problem q, int tiles_m, int tiles_n) {
        void *args[] = {&q, &tiles_m};
        return hipLaunchKernel(kernel, dim3(unsigned(tiles_m) * unsigned(tiles_n)), dim3(Cfg::kThreads), args, 0,
                               stream);
    });
}

// Split-K over a persistent grid ("stream-K" schedule), for products whose
// tiles would leave compute units idle or unevenly loaded. The product's
// work is the sequence of (tile, slab) iterations, tile after tile, each
// tile's slabs in K order; work-group w (numbered so that each XCD holds a
// contiguous run) takes iterations [w * per_wg, (w + 1) * per_wg), so every
// compute unit gets the same amount. A tile whose slabs all fall to one
// work-group is computed and stored as usual. A tile shared by several is
// computed in pieces: each work-group stores its unscaled partial tile in
// the workspace, and a second kernel adds a tile's partials in K order (so
// the result is the same on every run), scales, and updates C. Work-group w
// stores at most two partials: slot 2w for the piece its range starts with,
// slot 2w + 1 for the one it ends with.
struct SkPlan {
    int tiles_m, tiles_n;  // tile grid
    int slabs;             // slabs per tile, the partial one included
    int per_wg;            // iterations per work-group
    float *ws;             // 2 * grid partial tiles of BM * BN floats
};

template <class Cfg, bool TA, bool TB>
__global__ __launch_bounds__(Cfg::kThreads)
__attribute__((amdgpu_waves_per_eu(Cfg::kWavesPerEU, Cfg::kWavesPerEU))) void mfma_sk_kernel(Problem p, SkPlan sk)
{
    __shared__ __attribute__((aligned(16))) float lds[Tiles<Cfg, TA, TB>::kLdsFloats];
    constexpr int BM = Cfg::BM, BN = Cfg::BN;
    const int w = int(logical_workgroup(blockIdx.x, gridDim.x));
    const std::int64_t total = std::int64_t(sk.tiles_m) * sk.tiles_n * sk.slabs;
    const std::int64_t begin = std::int64_t(w) * sk.per_wg;
    const std::int64_t end = begin + sk.per_wg < total ? begin + sk.per_wg : total;
    for (std::int64_t it = begin; it < end;) {
        const std::int64_t t = it / sk.slabs;
        const int s0 = int(it - t * sk.slabs);
        const int s1 = end - t * sk.slabs < sk.slabs ? int(end - t * sk.slabs) : sk.slabs;
        int tm, tn;
        tile_of_index(unsigned(t), sk.tiles_m, unsigned(sk.tiles_n), Cfg::kGroupM, tm, tn);
        const bool whole = s0 == 0 && s1 == sk.slabs;
        const TileRange rg{s0, s1, whole ? nullptr : sk.ws + (2 * std::int64_t(w) + (it == begin ? 0 : 1)) * BM * BN};
        const bool edge = std::int64_t(tm + 1) * BM > p.M || std::int64_t(tn + 1) * BN > p.N;
        if (edge)
            interior_tile<Cfg, TA, TB, true, true>(p, tm, tn, lds, rg);
        else
            interior_tile<Cfg, TA, TB, false, true>(p, tm, tn, lds, rg);
        it = t * sk.slabs + s1;
        __syncthreads();  // the next piece reuses the LDS buffers
    }
}

// C <- alpha * (sum of a shared tile's partials, in K order) + beta * C, four
// consecutive columns per work-item; tile blockIdx.y (logical numbering).
template <int BM, int BN>
__global__ __launch_bounds__(256) void mfma_sk_fixup_kernel(Problem p, SkPlan sk)
{
    static_assert(BN % 4 == 0, "four columns per work-item");
    const int t = blockIdx.y;
    const std::int64_t first = std::int64_t(t) * sk.slabs, last = first + sk.slabs - 1;
    const int w0 = int(first / sk.per_wg), w1 = int(last / sk.per_wg);
    if (w0 == w1) return;  // stored whole by its work-group
    const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= BM * BN) return;
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int w = w0; w <= w1; ++w) {
        const std::int64_t slot = 2 * std::int64_t(w) + (std::int64_t(w) * sk.per_wg >= first ? 0 : 1);
        v += *reinterpret_cast<const f32x4 *>(sk.ws + slot * BM * BN + e);
    }
    int tm, tn;
    tile_of_index(unsigned(t), sk.tiles_m, unsigned(sk.tiles_n), SGEMM_MFMA_GROUP_M, tm, tn);
    const std::int64_t row = std::int64_t(tm) * BM + e / BN;
    const int col = tn * BN + e % BN;
    const float vals[4] = {v[0], v[1], v[2], v[3]};
    const bool inside = row < p.M && col + 4 <= p.N;
    update_n<4>(p.C, p.ldc, row, col, p.M, p.N, vals, inside, p.alpha, p.beta);
}

// Workspace bytes the split schedule of this configuration needs with `grid`
// work-groups.
template <class Cfg>
constexpr std::size_t sk_workspace_bytes(int grid)
{
    return std::size_t(2) * std::size_t(grid) * Cfg::BM * Cfg::BN * sizeof(float);
}

template <class Cfg, bool TA, bool TB>
hipError_t launch_sk(const Problem &p, float *ws, int grid, hipStream_t stream)
{
    SkPlan sk;
    sk.tiles_m = int((std::int64_t(p.M) + Cfg::BM - 1) / Cfg::BM);
    sk.tiles_n = int((std::int64_t(p.N) + Cfg::BN - 1) / Cfg::BN);
    sk.slabs = int((std::int64_t(p.K) + Cfg::BK - 1) / Cfg::BK);
    const std::int64_t total = std::int64_t(sk.tiles_m) * sk.tiles_n * sk.slabs;
    sk.per_wg = int((total + grid - 1) / grid);
    sk.ws = ws;
    Problem q = p;
    void *args[] = {&q, &sk};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&mfma_sk_kernel<Cfg, TA, TB>), dim3(grid),
                                   dim3(Cfg::kThreads), args, 0, stream);
    if (e != hipSuccess) return e;
    const unsigned per_tile = unsigned((Cfg::BM * Cfg::BN / 4 + 255) / 256);
    return hipLaunchKernel(reinterpret_cast<const void *>(&mfma_sk_fixup_kernel<Cfg::BM, Cfg::BN>),
                           dim3(per_tile, unsigned(sk.tiles_m * sk.tiles_n)), dim3(256), args, 0, stream);
}

// The split schedule with the tile shape the host chose.
template <bool TA, bool TB>
hipError_t launch_sk_by_tile(const Problem &p, MfmaTile tile, float *ws, int grid, hipStream_t stream)
{
    if (tile == MfmaTile::MidDual) return launch_sk<MidSplitCfg, TA, TB>(p, ws, grid, stream);
    return launch_sk<BigCfg, TA, TB>(p, ws, grid, stream);
}

// One launch with the tile shape the host chose for this product
// (select.cpp). The clamped reads of edge tiles need an FC operand (A
// transposed, B as given) at least 4 wide; narrower products take the
// general tiles, which guard every element.
template <bool TA, bool TB>
hipError_t launch_by_shape(const Problem &p, hipStream_t stream)
{
    if ((TA && p.M < 4) || (!TB && p.N < 4)) return launch_general<GeneralCfg, TA, TB>(p, stream);
    switch (p.tile) {
    case MfmaTile::Big: return launch_tiles<BigCfg, TA, TB>(p, stream);
    case MfmaTile::Mid: return launch_tiles<MidCfg, TA, TB>(p, stream);
    case MfmaTile::MidDual: return launch_tiles<MidDualCfg, TA, TB>(p, stream);
    case MfmaTile::Wide: return launch_tiles<WideCfg, TA, TB>(p, stream);
    case MfmaTile::WideN: return launch_tiles<WideNCfg, TA, TB>(p, stream);
    case MfmaTile::KSplit: return launch_ksplit<KSplitCfg, TA, TB>(p, stream);
    case MfmaTile::KSplit32: return launch_ksplit<KSplit32Cfg, TA, TB>(p, stream);
    // The tiles whose K range is split over their waves form buffer offsets
    // in 31 bits; larger operands take the LDS-staged tile of the same size
    // (two-set 64x64, eight-wave 128x128 for both larger ones).
    case MfmaTile::WSplit:
        if (wsplit_offsets_fit<Ws64Cfg>(p)) return launch_wsplit<Ws64Cfg, TA, TB>(p, stream);
        return launch_ksplit<KSplitCfg, TA, TB>(p, stream);
    case MfmaTile::WSplit96:
        if (wsplit_offsets_fit<Ws96Cfg>(p)) return launch_wsplit<Ws96Cfg, TA, TB>(p, stream);
        return launch_tiles<MidCfg, TA, TB>(p, stream);
    case MfmaTile::WSplit128:
        if (wsplit_offsets_fit<Ws128Cfg>(p)) return launch_wsplit<Ws128Cfg, TA, TB>(p, stream);
        return launch_tiles<MidCfg, TA, TB>(p, stream);
    case MfmaTile::Small: break;
    }
    return launch_tiles<SmallCfg, TA, TB>(p, stream);
}

}  // namespace
}  // namespace sgemm_impl

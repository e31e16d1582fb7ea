// Tile shapes of the matrix-core kernels, shared by the kernels (mfma.hpp)
// and the host-side choice of tile (select.cpp). Each is BM, BN, BK,
// WAVES_M, WAVES_N: a work-group computes a BM x BN tile of C with
// WAVES_M x WAVES_N waves, walking K in slabs of BK.
#pragma once

// General tiles (every element guarded): products whose operand stored with
// its free index contiguous (B as given, A transposed) is under 4 wide.
#ifndef SGEMM_MFMA_TILE
#define SGEMM_MFMA_TILE 128, 128, 32, 2, 4
#endif
// Tiles of the fast loop, largest first. The 256x256 and 128x128 tiles run eight
// waves (two per SIMD), so one wave's loads, LDS traffic and barrier waits
// overlap the other's matrix instructions; the 64x64 tile runs four, and so
// does the second 128x128 tile, of which two work-groups share a compute unit.
#ifndef SGEMM_MFMA_BIG_TILE
#define SGEMM_MFMA_BIG_TILE 256, 256, 16, 4, 2
#endif
#ifndef SGEMM_MFMA_MID_TILE
#define SGEMM_MFMA_MID_TILE 128, 128, 32, 2, 4
#endif
// The 128x128 tile of whole-tile launches stages two slabs in registers
// (loads issued two slabs before they are stored to LDS; +3-5% at 2048^3),
// which takes the register budget of one work-group per compute unit. The
// 256x256 tile has no room for a second set, and the 64x64 tile (four
// work-groups per compute unit) loses with one.
#ifndef SGEMM_MFMA_MID_REG_SETS
#define SGEMM_MFMA_MID_REG_SETS 2
#endif
// 128 x 128 tiles with 2 x 2 waves of 64 x 64, slabs of 16 and two staging
// register sets: four waves and 36 KB of LDS, so two work-groups share a
// compute unit, and one's loads, stores and barrier waits overlap the other's
// matrix instructions. Where a compute unit holds two or more 128 x 128
// tiles this beat the eight-wave tile above by 2-3% (interleaved medians on
// MI355X, TFLOP/s: 6144^3 143.4 -> 145.9, 4096 x 2048 x 4096 140.1 -> 143.3,
// 2048 x 4096 x 2048 136.9 -> 140.9); with one tile per compute unit it was
// level or up to 1.5% slower (2048^3), and slabs of 32 lost 7-9%. The split
// schedule's 128x128 pieces are this tile with one staging set.
#ifndef SGEMM_MFMA_MID_DUAL_TILE
#define SGEMM_MFMA_MID_DUAL_TILE 128, 128, 16, 2, 2
#endif
#ifndef SGEMM_MFMA_MID_DUAL_REG_SETS
#define SGEMM_MFMA_MID_DUAL_REG_SETS 2
#endif
// 192 x 128 tiles with 2 x 2 waves of 96 x 64, slabs of 16 and two staging
// register sets (47 KB of LDS; two work-groups fit a compute unit). Products
// whose 128 x 128 tiles would leave the compute units unevenly loaded but
// whose 192 x 128 tiles come out near a whole number per compute unit take
// them: 3001 x 2047 x 4093 (16 x 16 tiles) went from 116 to 132 TFLOP/s
// against the 64 x 64 tile, 3072 x 2048 x 4096 from 126 to 142 (interleaved
// medians on MI355X), with 2 x 4 waves of 96 x 32 and slabs of 32. The four
// waves then gained 1-3% where a compute unit holds one such tile (3001 x
// 2047 x 4093 135.3 -> 136.9, 3072 x 2048 x 4096 141.5 -> 143.6) and 3% where
// it holds several (6144^3 143.7 -> 148.1).
#ifndef SGEMM_MFMA_WIDE_TILE
#define SGEMM_MFMA_WIDE_TILE 192, 128, 16, 2, 2
#endif
#ifndef SGEMM_MFMA_WIDE_REG_SETS
#define SGEMM_MFMA_WIDE_REG_SETS 2
#endif
// The same tile turned round, 128 x 192 with 2 x 2 waves of 64 x 96, for
// products whose M and N are the other way round: 2047 x 3001 x 4093 takes
// 16 x 16 of them, one per compute unit, where it took 5.9 64 x 64 tiles per
// compute unit (four waves against eight of 32 x 96: 129.4 -> 133.5 TFLOP/s,
// 2048 x 3072 x 4096 137.9 -> 142.1).
#ifndef SGEMM_MFMA_WIDEN_TILE
#define SGEMM_MFMA_WIDEN_TILE 128, 192, 16, 2, 2
#endif
#ifndef SGEMM_MFMA_WIDEN_REG_SETS
#define SGEMM_MFMA_WIDEN_REG_SETS 2
#endif
// The small tiles take short slabs: BK = 16 here and 32 below measured 1-3.5%
// faster than 32 and 64 on every product that uses them, and twice as long
// lost 5-12%.
#ifndef SGEMM_MFMA_SMALL_TILE
#define SGEMM_MFMA_SMALL_TILE 64, 64, 16, 2, 2
#endif
// The small tile with its K range split over two sets of waves (BM, BN, BK,
// WAVES_M, WAVES_N, sets): two waves per SIMD where one small tile per
// compute unit would leave one.
#ifndef SGEMM_MFMA_KSPLIT_TILE
#define SGEMM_MFMA_KSPLIT_TILE 64, 64, 32, 2, 2, 2
#endif
// Staging register sets of that tile: slab t+1+sets is requested while slab t
// is multiplied. Two sets against one (interleaved medians on MI355X, TFLOP/s):
// 1024^3 92.6 -> 97.0, 1024 x 1024 x 4096 109.2 -> 117.5, 1000^3 81.6 -> 86.4,
// 896^3 72.8 -> 76.0; three and four sets gained less than two.
#ifndef SGEMM_MFMA_KSPLIT_REG_SETS
#define SGEMM_MFMA_KSPLIT_REG_SETS 2
#endif
// The same split over two sets of one wave each on 32 x 32 tiles, for the
// smallest products, which leave most compute units without a 64 x 64 tile
// (interleaved medians on MI355X, microseconds, 64 x 64 -> 32 x 32: 128^3
// 5.4 -> 4.5, 256^3 7.6 -> 5.7, 384^3 9.5 -> 6.4, 512^3 11.8 -> 7.9,
// 512 x 512 x 4096 70.1 -> 43.0; 768^3 16.7 -> 17.3 and 1024^3 22.3 -> 24.2
// stay on the 64 x 64 tiles).
#ifndef SGEMM_MFMA_KSPLIT32_TILE
#define SGEMM_MFMA_KSPLIT32_TILE 32, 32, 32, 1, 1, 2
#endif

// Tile rows per band of the tile order (tile_io.hpp: tile_of_index).
#ifndef SGEMM_MFMA_GROUP_M
#define SGEMM_MFMA_GROUP_M 8
#endif

namespace sgemm_impl {

// The tiles whose K range is split over their four waves, each wave holding
// the whole tile (wsplit.hpp): blocks of 32 x 32 per side (tile edge 64, 96,
// 128), k per chunk, register sets a wave's chunks stream through, and the
// waves per SIMD its registers are bounded for. The 64 x 64 tile keeps two
// sets within 256 registers, so two work-groups can share a compute unit;
// the larger ones take a compute unit each (their partial tiles fill most of
// the LDS anyway).
#ifndef SGEMM_MFMA_WSPLIT64
#define SGEMM_MFMA_WSPLIT64 2, 32, 2, 2
#endif
#ifndef SGEMM_MFMA_WSPLIT96
#define SGEMM_MFMA_WSPLIT96 3, 32, 2, 1
#endif
#ifndef SGEMM_MFMA_WSPLIT128
#define SGEMM_MFMA_WSPLIT128 4, 16, 2, 1
#endif

// Interior tile shape of one matrix-core launch. WSplit, WSplit96 and
// WSplit128 are the tiles whose K range is split over their waves.
enum class MfmaTile { Big, Mid, Small, KSplit, Wide, WideN, MidDual, KSplit32, WSplit, WSplit96, WSplit128 };

namespace tiles {
constexpr int kGeneral[] = {SGEMM_MFMA_TILE};
constexpr int kBig[] = {SGEMM_MFMA_BIG_TILE};
constexpr int kMid[] = {SGEMM_MFMA_MID_TILE};
constexpr int kSmall[] = {SGEMM_MFMA_SMALL_TILE};
constexpr int kKSplit[] = {SGEMM_MFMA_KSPLIT_TILE};
constexpr int kWide[] = {SGEMM_MFMA_WIDE_TILE};
constexpr int kWideN[] = {SGEMM_MFMA_WIDEN_TILE};
constexpr int kMidDual[] = {SGEMM_MFMA_MID_DUAL_TILE};
constexpr int kKSplit32[] = {SGEMM_MFMA_KSPLIT32_TILE};
// BM, BN, k per chunk, 1 x 1 waves per set, 4 sets (each wave one set).
constexpr int kWs64[] = {SGEMM_MFMA_WSPLIT64};
constexpr int kWs96[] = {SGEMM_MFMA_WSPLIT96};
constexpr int kWs128[] = {SGEMM_MFMA_WSPLIT128};
constexpr int kWSplit[] = {32 * kWs64[0], 32 * kWs64[0], kWs64[1], 1, 1, 4};
constexpr int kWSplit96[] = {32 * kWs96[0], 32 * kWs96[0], kWs96[1], 1, 1, 4};
constexpr int kWSplit128[] = {32 * kWs128[0], 32 * kWs128[0], kWs128[1], 1, 1, 4};
}  // namespace tiles

}  // namespace sgemm_impl

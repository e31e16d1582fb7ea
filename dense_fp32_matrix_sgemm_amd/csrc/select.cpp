// Shape-aware choice of the matrix-core tile ("Matrix Multiplication --
// Naive to Tiled", section 07 and exercise 2: tile sizes are tuned per
// problem; here the library chooses among the tile shapes it carries).
//
// One launch covers C with ceil(M/BM) x ceil(N/BN) tiles of one shape (edge
// tiles run the same loop as the others). Every work-group keeps a compute
// unit's matrix cores busy for its whole K loop, so the launch takes as long
// as the busiest compute unit: with n tiles over CUs compute units it holds
// m = ceil(n / CUs) tiles, run up to `slots` at a time. A batch of q
// concurrent tiles takes q * BM * BN / rate(q), in units where one 256x256
// tile per compute unit runs at rate 1; more concurrent tiles per compute
// unit hide more latency, so rate grows with q. The rates are measured on
// MI355X with each shape forced over a set of products (TFLOP/s over 256
// compute units, relative to 147 for 256x256 at 4096^3): 128x128 0.91, one
// at a time (its two staging register sets leave room for one work-group);
// 128x128 in four waves 0.89 alone and 0.925 two at a time (two such
// work-groups share a compute unit; 2-3% ahead of the eight-wave 128x128
// tile wherever a compute unit holds two or more, level or behind with one);
// 192x128 0.93, one at a time (0.92-0.96 on products it tiles exactly),
// and 128x192, the same tile turned round, likewise;
// 64x64 0.59, 0.72, 0.79 and 0.84 for one to four;
// 64x64 with its K range split over two sets of waves 0.65 alone and 0.78 two
// at a time (it takes 1024^3 from 80 to 95 TFLOP/s); 32x32 split the same way
// over two single waves 0.25, 0.30, 0.40 and 0.50 for one to four (fitted so
// that it takes the products that give each compute unit at most one such
// tile: 128^3 to 512^3, 300 x 257 x 513 and 512 x 512 x 4096 ran 17-63%
// faster on it; with two per compute unit 700^3 and 1000 x 300 x 1000 ran
// 8-10% slower, and 768^3 and 1024^3 3-8% slower). (A 256x128 shape
// measured 0.85-0.94 alone and never beat these.) The 64x64 rates predate
// those tiles' shorter slabs, which made both 2-4% faster; with the kernels
// as they are, a forced-shape run of 14 products found this choice within 1%
// of the fastest shape on every one. The 64x64 tile whose K range is split
// over its four waves (wsplit.hpp) runs at 0.75 alone (1024^3: 111 TFLOP/s)
// and 0.82 two at a time (2048 x 1024 x 1024: 121), ahead of the two-set
// tile wherever either would be chosen (interleaved medians on MI355X,
// TFLOP/s, two-set -> four-wave split: 1024^3 102.6 -> 111.2, 1000^3 89.9 ->
// 94.4, 768^3 54.9 -> 58.6, 2048 x 1024 x 1024 116.0 -> 121.0, 1536^3 90.3
// -> 95.9); it loses where it gives most compute units no tile at all
// (512 x 512 x 4096: 49.4 on the 32x32 tile, 31.9 on it), and where a compute
// unit holds three or more (2048^3: 116 against 135 for 128x128). The same
// split on 96x96 and 128x128 tiles, one work-group per compute unit, runs at
// 0.89 and 1.02 where it is taken (1536^3 89.7 -> 131.3,
// 1536 x 1536 x 4096 92.3 -> 143.0, 2048^3 135.4 -> 143.1, 2048^2 x 4096
// 138.9 -> 147.7, 1920^3 119.6 -> 125.5; forced where it would hold more,
// 96x96 at 2048^3 117 and 128x128 at 1536^3 80).
//
// Pure C++ (no HIP), so it is tested on the host.
#include <cstddef>
#include <cstdint>

#include "select.hpp"
#include "sgemm.h"

namespace sgemm_impl {
namespace {

struct Candidate {
    MfmaTile tile;
    int bm, bn;
    int slots;           // tiles a compute unit runs at once
    double rate[4];      // rate with 1..slots tiles resident
};

std::int64_t ceil_div(std::int64_t a, std::int64_t b) { return (a + b - 1) / b; }

double launch_time(const Candidate &c, std::int64_t M, std::int64_t N, std::int64_t cus)
{
    const std::int64_t m = ceil_div(ceil_div(M, c.bm) * ceil_div(N, c.bn), cus);
    const double work = double(c.bm) * c.bn;
    const std::int64_t full = m / c.slots, rest = m % c.slots;
    double t = double(full) * c.slots * work / c.rate[c.slots - 1];
    if (rest > 0) t += double(rest) * work / c.rate[rest - 1];
    return t;
}

const Candidate kCandidates[] = {
    {MfmaTile::Big, tiles::kBig[0], tiles::kBig[1], 1, {1.0, 0, 0, 0}},
    {MfmaTile::Mid, tiles::kMid[0], tiles::kMid[1], 1, {0.91, 0, 0, 0}},
    {MfmaTile::MidDual, tiles::kMidDual[0], tiles::kMidDual[1], 2, {0.89, 0.925, 0, 0}},
    {MfmaTile::Wide, tiles::kWide[0], tiles::kWide[1], 1, {0.93, 0, 0, 0}},
    {MfmaTile::WideN, tiles::kWideN[0], tiles::kWideN[1], 1, {0.93, 0, 0, 0}},
    {MfmaTile::Small, tiles::kSmall[0], tiles::kSmall[1], 4, {0.59, 0.72, 0.79, 0.84}},
    {MfmaTile::KSplit, tiles::kKSplit[0], tiles::kKSplit[1], 2, {0.65, 0.78, 0, 0}},
    {MfmaTile::KSplit32, tiles::kKSplit32[0], tiles::kKSplit32[1], 4, {0.25, 0.30, 0.40, 0.50}},
    {MfmaTile::WSplit, tiles::kWSplit[0], tiles::kWSplit[1], 2, {0.75, 0.82, 0, 0}},
    {MfmaTile::WSplit96, tiles::kWSplit96[0], tiles::kWSplit96[1], 1, {0.89, 0, 0, 0}},
    {MfmaTile::WSplit128, tiles::kWSplit128[0], tiles::kWSplit128[1], 1, {1.02, 0, 0, 0}},
};

}  // namespace

// Whether the 64x64 tile with its K range split over its four waves may take
// the product. It runs two work-groups per compute unit, so a third tile per
// compute unit waits for a second round, and the partial last chunk of a
// ragged K (not a multiple of 32) costs each tile a load's round trip. Where
// both count, the 64x64 tiles that hold three or four per compute unit at
// once were faster (interleaved medians on MI355X, TFLOP/s, split over waves
// against plain 64x64: 1200 x 2400 x 1200 86.1 / 106.0, 1536 x 1500 x 1000
// 70.4 / 82.7), and so they were with more than three per compute unit
// (2200^3 99.5 / 112.2, 2200^2 x 2208 110.2 / 113.5); with up to two per
// compute unit whatever K, or three with K a multiple of 32, this tile was
// faster (1000^3 96.6 / 74.5, 1536^3 95.7 / 90.6, 1200^3 80.3 / 77.6 before,
// 2048 x 1024 x 1000 118.0 / 109.3 on the two-set tile, 80 x 12000 x 1000
// 55.6 / 50.7). A product under 64 wide leaves most of the tile idle (16000
// x 8 x 1000: 10.0 against 11.0 on the 32x32 tile).
bool wsplit_fits(std::int64_t M, std::int64_t N, std::int64_t K, std::int64_t cus)
{
    if (M < 64 || N < 64) return false;
    const std::int64_t m = ceil_div(ceil_div(M, 64) * ceil_div(N, 64), cus);
    return m <= 2 || (K % 32 == 0 && m <= 3);
}

// The 96x96 and 128x128 tiles split over their waves run one work-group per
// compute unit, so a compute unit's tiles run one after another, each paying
// its first loads and its sum of partial tiles with nothing to overlap them
// (about 7 us a tile; the 128x128 tile's loop runs at 0.98 of peak against
// 0.95 for the 256x256 tile). So they are taken where a compute unit holds a
// single one; the 128x128 tile also where K >= 2048 and its tiles fill every
// round of the compute units to 95% or more (4096^3 147.5 -> 150.3,
// 6144^2 x 4096 147.3 -> 150.3, 8192^2 x 4096 147.9 -> 150.7, 16384 x 512 x
// 4096 142.4 -> 148.3, 2048 x 4096 x 2048 141.5 -> 145.3; not at 4096^2 x
// 1024, 138.0 against 140.4, 5000 x 3000 x 2000, 94% full, 122.9 against
// 125.0, or 3072^3, 75%, 112 against 127). Not for products narrower than
// the tile.
bool wsplit_large_fits(std::int64_t M, std::int64_t N, std::int64_t K, std::int64_t edge, std::int64_t cus)
{
    if (M < edge || N < edge) return false;
    const std::int64_t tiles = ceil_div(M, edge) * ceil_div(N, edge);
    const std::int64_t m = ceil_div(tiles, cus);
    if (m == 1) return true;
    return edge == 128 && K >= 2048 && tiles * 20 >= m * cus * 19;
}

MfmaTile choose_mfma_tile(int M, int N, int K, int cus)
{
#if defined(SGEMM_MFMA_FORCE_TILE)
    // Tile sweeps: every product takes the shape numbered here (MfmaTile).
    (void)M;
    (void)N;
    (void)K;
    (void)cus;
    return static_cast<MfmaTile>(SGEMM_MFMA_FORCE_TILE);
#endif
    const std::int64_t n_cus = cus > 0 ? cus : 256;
    MfmaTile best = MfmaTile::Big;
    double best_t = -1.0;
    for (const Candidate &c : kCandidates) {  // ties go to the earlier (larger or simpler) shape
        if (c.tile == MfmaTile::WSplit && !wsplit_fits(M, N, K, n_cus)) continue;
        if ((c.tile == MfmaTile::WSplit96 || c.tile == MfmaTile::WSplit128) &&
            !wsplit_large_fits(M, N, K, c.bm, n_cus))
            continue;
        const double t = launch_time(c, M, N, n_cus);
        if (best_t < 0.0 || t < best_t) {
            best_t = t;
            best = c.tile;
        }
    }
    return best;
}

// Split schedule. Times in seconds, from the same measured rates: rate 1 is
// 147 TFLOP/s over 256 compute units. Work-group w of `grid` takes
// ceil(tiles * slabs / grid) iterations of BM x BN x BK; a compute unit
// runs `slots` work-groups at once at `rate`. Tiles shared by several
// work-groups cost their partials' round trip (written, then read by the
// second kernel) and that kernel's launch. The rates and the partials'
// bandwidth (they mostly stay in the 256 MB Infinity Cache) are fitted to
// forced-schedule runs on MI355X: 256x256 pieces 0.93, 128x128 pieces two at
// a time 0.85 (3001 x 2047 x 4093, 3072 x 2048 x 4096, 2560^3, 1536^3). The
// 128x128 pieces have since moved to the four-wave tile, 4-6% faster; the
// model keeps the rate it was fitted with, so it splits no more products
// than before.
namespace {

constexpr double kRate1PerCu = 147e12 / 256;  // FLOP/s of one compute unit at rate 1
constexpr double kPartialBytesPerS = 8e12;    // the partials' write and read
constexpr double kSecondLaunchS = 4e-6;       // the adding kernel's launch and ramp

struct SplitCandidate {
    MfmaTile tile;
    int bm, bn, bk;
    int slots;
    double rate;
};

double split_time(const SplitCandidate &c, std::int64_t M, std::int64_t N, std::int64_t K, int cus, int grid)
{
    const std::int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
    const std::int64_t slabs = ceil_div(K, c.bk);
    const std::int64_t per_wg = ceil_div(tiles * slabs, grid);
    const double wg_flop = double(per_wg) * c.bm * c.bn * c.bk * 2.0;
    double t = double(c.slots) * wg_flop / (kRate1PerCu * c.rate);
    (void)cus;
    // Pieces of shared tiles: tile t spans work-groups [t*slabs/per_wg, ((t+1)*slabs-1)/per_wg].
    std::int64_t pieces = 0;
    for (std::int64_t t0 = 0; t0 < tiles; ++t0) {
        const std::int64_t w0 = (t0 * slabs) / per_wg, w1 = ((t0 + 1) * slabs - 1) / per_wg;
        if (w1 > w0) pieces += w1 - w0 + 1;
    }
    if (pieces > 0) t += 2.0 * double(pieces) * c.bm * c.bn * 4.0 / kPartialBytesPerS + kSecondLaunchS;
    return t;
}

}  // namespace

std::size_t split_workspace_bytes(MfmaTile tile, int grid)
{
    const int *d = tile == MfmaTile::MidDual ? tiles::kMidDual : tiles::kBig;
    return std::size_t(2) * std::size_t(grid > 0 ? grid : 0) * std::size_t(d[0]) * std::size_t(d[1]) * sizeof(float);
}

SplitChoice choose_split(int M, int N, int K, int cus)
{
    using namespace tiles;
    SplitChoice none{false, MfmaTile::Big, 0, 0};
    if (M <= 0 || N <= 0 || K <= 0) return none;
    const int n_cus = cus > 0 ? cus : 256;
    constexpr int kMaxCus = 1 << 16;  // no device has more; keeps the grid (CUs x slots) in range
    if (n_cus > kMaxCus) return none;
    // Whole tiles: the chosen shape's estimated time.
    const MfmaTile dp_tile = choose_mfma_tile(M, N, K, n_cus);
    const Candidate *dp = &kCandidates[0];
    for (const Candidate &c : kCandidates)
        if (c.tile == dp_tile) dp = &c;
    const double t_dp = launch_time(*dp, M, N, n_cus) * 2.0 * double(K) / kRate1PerCu;

    const SplitCandidate splits[] = {
        {MfmaTile::Big, kBig[0], kBig[1], kBig[2], 1, 0.93},
        {MfmaTile::MidDual, kMidDual[0], kMidDual[1], kMidDual[2], 2, 0.85},
    };
    SplitChoice best = none;
    double best_t = 0.97 * t_dp;  // the split schedule must win by a margin
    for (const SplitCandidate &c : splits) {
        const int grid = n_cus * c.slots;
        const std::int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
        if (tiles > 65535) continue;  // the adding kernel's grid rows
        const double t = split_time(c, M, N, K, n_cus, grid);
        if (t < best_t) {
            best_t = t;
            best = {true, c.tile, grid, split_workspace_bytes(c.tile, grid)};
        }
    }
    return best;
}

// The register-blocked rung's tile: the pages' 128 x 128 where C holds at
// least one and a half of them per compute unit, else 64 x 64 where it holds
// at least one per two compute units, else 32 x 32 where it holds at least
// one of those per two compute units, else 16 x 16. Measured on MI355X with
// each tile forced (back-to-back launches, microseconds, 128 / 64 / 32):
// 512^3 91 / 32 / 18; 1024^3 198 / 67 / 87; 1536^3 301 / 228 / 251; 2048^3
// 398 / 301 / 567; 3001 x 2047 x 4093 905 / 963 / 1684; 4096^3 1669 / 2179 /
// 4370. One 128 x 128 tile per compute unit (2048^3) leaves one wave per SIMD
// with nothing to hide its latencies behind, so there the 64 x 64 tile's four
// per compute unit win. 32 / 16: 128^3 6.0 / 3.9; 256^3 9.9 / 5.7; 300 x 257
// x 513 19.7 / 15.3; 384^3 14.3 / 14.5; 512^3 18.3 / 23.6.
int regblock_tile_size(int M, int N, int cus)
{
#if defined(SGEMM_REGBLOCK_FORCE_TILE)
    (void)M;
    (void)N;
    (void)cus;
    return SGEMM_REGBLOCK_FORCE_TILE;
#else
    const std::int64_t n_cus = cus > 0 ? cus : 256;
    auto tiles = [&](int t) { return ceil_div(M, t) * ceil_div(N, t); };
    if (2 * tiles(128) >= 3 * n_cus) return 128;
    if (2 * tiles(64) >= n_cus) return 64;
    if (2 * tiles(32) >= n_cus) return 32;
    return 16;
#endif
}

}  // namespace sgemm_impl

extern "C" int sgemm_regblock_tile(int M, int N, int cus)
{
    if (M < 0 || N < 0) return SGEMM_ERR_DIM;
    return sgemm_impl::regblock_tile_size(M, N, cus);
}

extern "C" int sgemm_mfma_tile(int M, int N, int K, int cus, int *BM, int *BN)
{
    using namespace sgemm_impl;
    if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_DIM;
    if (BM == nullptr || BN == nullptr) return SGEMM_ERR_NULL;
    const int *dims = tiles::kSmall;
    switch (choose_mfma_tile(M, N, K, cus)) {
    case MfmaTile::Big: dims = tiles::kBig; break;
    case MfmaTile::Mid: dims = tiles::kMid; break;
    case MfmaTile::Small: dims = tiles::kSmall; break;
    case MfmaTile::KSplit: dims = tiles::kKSplit; break;
    case MfmaTile::Wide: dims = tiles::kWide; break;
    case MfmaTile::WideN: dims = tiles::kWideN; break;
    case MfmaTile::MidDual: dims = tiles::kMidDual; break;
    case MfmaTile::KSplit32: dims = tiles::kKSplit32; break;
    case MfmaTile::WSplit: dims = tiles::kWSplit; break;
    case MfmaTile::WSplit96: dims = tiles::kWSplit96; break;
    case MfmaTile::WSplit128: dims = tiles::kWSplit128; break;
    }
    *BM = dims[0];
    *BN = dims[1];
    return SGEMM_OK;
}

extern "C" std::size_t sgemm_ex_workspace_size(int transA, int transB, int M, int N, int K, int cus)
{
    using namespace sgemm_impl;
    const bool ok_op = (transA == SGEMM_OP_N || transA == SGEMM_OP_T) && (transB == SGEMM_OP_N || transB == SGEMM_OP_T);
    if (!ok_op || M <= 0 || N <= 0 || K <= 0) return 0;
    // Products whose free-index-contiguous operand is under 4 wide take the
    // general tiles, never the split schedule.
    if ((transA == SGEMM_OP_T && M < 4) || (transB == SGEMM_OP_N && N < 4)) return 0;
    const SplitChoice c = choose_split(M, N, K, cus);
    return c.use ? c.bytes : 0;
}

extern "C" int sgemm_mfma_shape(int M, int N, int K, int cus, int *shape)
{
    using namespace sgemm_impl;
    if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_DIM;
    if (shape == nullptr) return SGEMM_ERR_NULL;
    const int *dims = tiles::kSmall;
    int sets = 1;
    switch (choose_mfma_tile(M, N, K, cus)) {
    case MfmaTile::Big: dims = tiles::kBig; break;
    case MfmaTile::Mid: dims = tiles::kMid; break;
    case MfmaTile::Small: dims = tiles::kSmall; break;
    case MfmaTile::KSplit:
        dims = tiles::kKSplit;
        sets = tiles::kKSplit[5];
        break;
    case MfmaTile::KSplit32:
        dims = tiles::kKSplit32;
        sets = tiles::kKSplit32[5];
        break;
    case MfmaTile::WSplit:
        dims = tiles::kWSplit;
        sets = tiles::kWSplit[5];
        break;
    case MfmaTile::WSplit96:
        dims = tiles::kWSplit96;
        sets = tiles::kWSplit96[5];
        break;
    case MfmaTile::WSplit128:
        dims = tiles::kWSplit128;
        sets = tiles::kWSplit128[5];
        break;
    case MfmaTile::Wide: dims = tiles::kWide; break;
    case MfmaTile::WideN: dims = tiles::kWideN; break;
    case MfmaTile::MidDual: dims = tiles::kMidDual; break;
    }
    for (int i = 0; i < 5; ++i) shape[i] = dims[i];
    shape[5] = sets;
    return SGEMM_OK;
}

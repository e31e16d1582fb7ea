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
// compute units, relative to 147 for 256x256 at 4096^3): 128x128 0.88 alone
// and 0.93 two at a time; 64x64 0.59, 0.72, 0.79 and 0.84 for one to four.
// (A 256x128 shape measured 0.85-0.94 alone and never beat these three.)
//
// Pure C++ (no HIP), so it is tested on the host.
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

}  // namespace

MfmaTile choose_mfma_tile(int M, int N, int cus)
{
    using namespace tiles;
    const Candidate cands[] = {
        {MfmaTile::Big, kBig[0], kBig[1], 1, {1.0, 0, 0, 0}},
        {MfmaTile::Mid, kMid[0], kMid[1], 2, {0.88, 0.93, 0, 0}},
        {MfmaTile::Small, kSmall[0], kSmall[1], 4, {0.59, 0.72, 0.79, 0.84}},
    };
    const std::int64_t n_cus = cus > 0 ? cus : 256;
    MfmaTile best = MfmaTile::Big;
    double best_t = -1.0;
    for (const Candidate &c : cands) {  // ties go to the larger tile (less traffic)
        const double t = launch_time(c, M, N, n_cus);
        if (best_t < 0.0 || t < best_t) {
            best_t = t;
            best = c.tile;
        }
    }
    return best;
}

}  // namespace sgemm_impl

extern "C" int sgemm_mfma_tile(int M, int N, int cus, int *BM, int *BN)
{
    using namespace sgemm_impl;
    if (M < 0 || N < 0) return SGEMM_ERR_DIM;
    if (BM == nullptr || BN == nullptr) return SGEMM_ERR_NULL;
    const int *dims = tiles::kSmall;
    switch (choose_mfma_tile(M, N, cus)) {
    case MfmaTile::Big: dims = tiles::kBig; break;
    case MfmaTile::Mid: dims = tiles::kMid; break;
    case MfmaTile::Small: dims = tiles::kSmall; break;
    }
    *BM = dims[0];
    *BN = dims[1];
    return SGEMM_OK;
}

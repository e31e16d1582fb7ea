// Host-side choice of the matrix-core launch shape (pure C++).
#pragma once

#include <cstddef>

#include "tiles.hpp"

namespace sgemm_impl {

// The interior tile shape with the smallest estimated time for an M x N x K
// product on `cus` compute units (cus <= 0 means 256, an MI355X). K matters
// only to the 64x64 tile whose K range is split over its waves.
MfmaTile choose_mfma_tile(int M, int N, int K, int cus);

// The split ("stream-K") schedule for an M x N x K product: whether its
// estimated time beats the whole-tile launch, the tile shape and work-group
// count it would use, and the workspace it needs then (0 when not used).
struct SplitChoice {
    bool use;
    MfmaTile tile;
    int grid;
    std::size_t bytes;
};
SplitChoice choose_split(int M, int N, int K, int cus);

// Workspace of the split schedule: two partial tiles per work-group.
std::size_t split_workspace_bytes(MfmaTile tile, int grid);

// Edge of the square tile (128, 64 or 32) the register-blocked rung takes
// for an M x N product on `cus` compute units (cus <= 0 means 256).
int regblock_tile_size(int M, int N, int cus);

// Size of the library's own static scratch buffer (sgemm_ex_noalloc): the
// largest workspace the split schedule asks for on a 256-CU MI355X (one
// 256 x 256 work-group per compute unit, two partial tiles each).
constexpr std::size_t kNoallocScratchBytes = std::size_t(128) << 20;

}  // namespace sgemm_impl

// Host-side choice of the matrix-core launch shape (pure C++).
#pragma once

#include "tiles.hpp"

namespace sgemm_impl {

// The interior tile shape with the smallest estimated time for an M x N
// product on `cus` compute units (cus <= 0 means 256, an MI355X).
MfmaTile choose_mfma_tile(int M, int N, int cus);

}  // namespace sgemm_impl

// Tile scheduling shared by the GEMM kernels.
#pragma once

#include "common.hpp"

namespace qlq {

// Map a linear block id to a (tile_m, tile_n) pair.
//
// Workgroups are dealt round-robin to the 8 XCDs (block id mod 8), and each
// XCD has its own L2.  When the tile count is a multiple of 8, block id `pid`
// is remapped so that each XCD receives one contiguous range of tiles; inside
// that range tiles go in groups of GROUP_M tile-rows, so the blocks an XCD
// runs at the same time share A panels (same m) and B panels (same n) in its
// L2.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  int t = pid;
  if ((T & 7) == 0) t = (pid & 7) * (T >> 3) + (pid >> 3);
  const int per_group = GROUP_M * tiles_n;
  const int group = t / per_group;
  const int first_m = group * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int r = t - group * per_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

}  // namespace qlq

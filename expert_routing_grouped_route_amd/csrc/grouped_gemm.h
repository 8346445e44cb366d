// Tile space shared by the grouped GEMM kernels (bf16 and fp32).
//
// M-tiles of kBM = 256 rows per expert come from the tile table that the
// dispatch scan writes (tile_off[e] = M-tiles of the experts before e).
// For the fp32 kernels (routed_tile below) the tiles of an expert run n-tile
// outer, m-tile inner, so the tiles that share a weight slice are adjacent;
// the bf16 kernels use a grouped raster of their own (gemm_bf16.hip).  The
// grid is sized by an upper bound of the routed tiles (no host read-back of
// the counts); slots past the device-side count return at once.
// Shared-expert tiles follow the routed slots.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// Routed tile L -> expert e, m-tile m, n-tile n; false when L is past the
// device-side tile count.
__device__ __forceinline__ bool routed_tile(int L, const int32_t* __restrict__ tile_off, int E,
                                            int nt, int& e, int& m, int& n) {
  const int total = tile_off[E] * nt;
  if (L >= total) return false;
  int lo = 0, hi = E - 1;  // largest e with tile_off[e] * nt <= L (an expert with tiles)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_off[mid] * nt <= L) lo = mid;
    else hi = mid - 1;
  }
  e = lo;
  const int mt = tile_off[e + 1] - tile_off[e];
  const int local = L - tile_off[e] * nt;
  n = local / mt;
  m = local - n * mt;
  return true;
}

// Grid of one grouped GEMM launch.
struct GemmGrid {
  int mtb;         // upper bound of the routed M-tiles
  int nt_r;        // n-tiles per routed expert
  int nt_s;        // n-tiles per shared expert
  int mt_s;        // m-tiles over the T rows of the shared experts
  int n_shared;    // shared-expert tiles
  int64_t routed;  // routed tile slots (an upper bound)
  int64_t total;   // all slots (routed + shared), before any padding
  int run = 8;     // bf16 kernels: consecutive works per XCD run
  int gm = 4;      // bf16 kernels: m-tiles per group of the tile raster
};

}  // namespace moe

// Tile schedule of the grouped expert GEMMs: M-tiles are numbered expert by expert from
// the device-side row offsets, so a kernel launched for the worst case finds its own work.
#pragma once

#include "common.hpp"

namespace moe {

// Maps M-tile id `tile` to (expert, first row, rows in tile). Every wave computes the same
// answer independently. Returns false past the last tile.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int BM,
                                          int tile, int& e_out, int& row0, int& rows) {
  const int lane = lane_id();
  int n[4], tiles[4], mine = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * lane + q;
    n[q] = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    tiles[q] = (n[q] + BM - 1) / BM;
    mine += tiles[q];
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  const int excl = incl - mine;
  const unsigned long long own = __ballot(tile >= excl && tile < incl);
  if (own == 0ull) return false;
  const int owner = __ffsll((long long)own) - 1;
  int e = -1, mt = 0;
  int run = excl;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (e < 0 && tile < run + tiles[q]) {
      e = 4 * lane + q;
      mt = tile - run;
    }
    run += tiles[q];
  }
  e = __shfl(e, owner);
  mt = __shfl(mt, owner);
  const int start = offsets[e] + mt * BM;
  e_out = e;
  row0 = start;
  rows = min(BM, offsets[e + 1] - start);
  return true;
}

}  // namespace moe

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

// Tiles of a grouped GEMM laid out as (M-tiles x nt column tiles) per expert, experts in
// order; within an expert the tiles go in blocks of at most mb M-tiles by nb column tiles
// (M-blocks outer, then column blocks, then the M-tiles fastest). A block (mb x nb tiles) is
// about as many tiles as one XCD runs at once, so concurrent tiles share both their row
// panels and their column panels in that XCD's L2, however many M-tiles the expert has. tile_scan takes the per-expert tile counts (every wave computes the same);
// tile_of maps a linear tile id to (expert, first row, rows, column tile).
struct TileScan {
  int excl, incl;  // this lane's experts (4 lane, .. 4 lane + 3): first tile id, one past last
  int total;       // tiles of all experts
  int tiles[4];
};

__device__ __forceinline__ TileScan tile_scan(const int32_t* __restrict__ offsets, int E, int BM,
                                              int nt) {
  const int lane = lane_id();
  TileScan sc;
  int mine = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * lane + q;
    const int n = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    sc.tiles[q] = ((n + BM - 1) / BM) * nt;
    mine += sc.tiles[q];
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  sc.incl = incl;
  sc.excl = incl - mine;
  sc.total = __shfl(incl, kWave - 1);
  return sc;
}

__device__ __forceinline__ void tile_of(const TileScan& sc, const int32_t* __restrict__ offsets,
                                        int BM, int nt, int mb, int nb, int L, int& e_out,
                                        int& row0, int& rows, int& n_tile) {
  const int lane = lane_id();
  const unsigned long long own = __ballot(L >= sc.excl && L < sc.incl);
  const int owner = __ffsll((long long)own) - 1;
  int e = -1, local = 0;
  int run = sc.excl;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (e < 0 && L < run + sc.tiles[q]) {
      e = 4 * lane + q;
      local = L - run;
    }
    run += sc.tiles[q];
  }
  e = __shfl(e, owner);
  local = __shfl(local, owner);
  const int cnt = offsets[e + 1] - offsets[e];
  const int tm = (cnt + BM - 1) / BM;  // M-tiles of this expert
  const int mbe = min(mb, tm);           // (so mbe * nt <= tm * nt, the expert's tiles)
  const int mblk = local / (mbe * nt);   // every M-block but the last has mbe M-tiles
  const int mj = min(mbe, tm - mblk * mbe);
  const int rem = local - mblk * mbe * nt;
  const int blk = rem / (mj * nb);
  const int within = rem - blk * mj * nb;
  const int m = mblk * mbe + within % mj;
  n_tile = blk * nb + within / mj;
  e_out = e;
  row0 = offsets[e] + m * BM;
  rows = min(BM, cnt - m * BM);
}

}  // namespace moe

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

// Maps block b of a grid of at least (real tile count rounded up to 8) blocks to a tile
// (expert, first row, rows, column tile) of the (M-tiles x nt column tiles) grid of each
// expert. Experts come in order; within an expert the
// tiles go in blocks of nb column tiles, and inside a block the M-tiles vary fastest. A
// block of one expert (its M-tiles x nb column tiles) is about as many tiles as one XCD runs
// at once, so concurrent blocks share both their activation rows and their weight columns
// in that XCD's L2. Every wave computes the same answer. Returns false past the last tile.
__device__ __forceinline__ bool find_tile_2d(const int32_t* __restrict__ offsets, int E, int BM,
                                             int nt, int nb, int b, int& e_out, int& row0,
                                             int& rows, int& n_tile) {
  const int lane = lane_id();
  int n[4], tiles[4], mine = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * lane + q;
    n[q] = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    tiles[q] = ((n[q] + BM - 1) / BM) * nt;
    mine += tiles[q];
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  const int excl = incl - mine;
  // Block b runs on XCD b % 8; each XCD takes one contiguous eighth of the real tiles.
  const int total = __shfl(incl, kWave - 1);
  const int chunk = (total + 7) >> 3;
  if ((b >> 3) >= chunk) return false;
  const int L = (b & 7) * chunk + (b >> 3);
  const unsigned long long own = __ballot(L >= excl && L < incl);
  if (own == 0ull) return false;
  const int owner = __ffsll((long long)own) - 1;
  int e = -1, local = 0;
  int run = excl;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (e < 0 && L < run + tiles[q]) {
      e = 4 * lane + q;
      local = L - run;
    }
    run += tiles[q];
  }
  e = __shfl(e, owner);
  local = __shfl(local, owner);
  const int cnt = offsets[e + 1] - offsets[e];
  const int tm = (cnt + BM - 1) / BM;  // M-tiles of this expert
  const int blk = local / (tm * nb);
  const int within = local - blk * tm * nb;
  const int m = within % tm;
  n_tile = blk * nb + within / tm;
  e_out = e;
  row0 = offsets[e] + m * BM;
  rows = min(BM, cnt - m * BM);
  return true;
}

}  // namespace moe

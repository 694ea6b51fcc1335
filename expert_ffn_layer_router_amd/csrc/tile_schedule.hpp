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
// about as many tiles as one XCD runs at once, so concurrent tiles share both their row panels
// and their column panels in that XCD's L2, however many M-tiles the expert has.
// With `short_last`, each expert's last tile when it has at most 128 rows (a short tile: the
// kernel runs it with half or a quarter of the MFMAs) is taken out of that order and put in a
// second run after all the others, experts in order, column tiles in order. A launch whose
// split-K tail can hold every short tile asks for this, so the short tiles become the tail and
// every block's whole tiles cost the same; elsewhere it does not, since a short tile at the
// end no longer shares its column panel with the tiles beside it. tile_scan takes the
// per-expert tile counts (every wave computes the same); tile_of maps a linear tile id to
// (expert, first row, rows, column tile).
constexpr int kShortRows = 128;  // a last M-tile with at most this many rows is short

struct TileScan {
  int excl, incl;  // this lane's experts (4 lane .. 4 lane + 3), short tiles left out: first
                   // tile id, one past the last
  int sexcl;       // the short tiles of the experts before this lane's
  int sbits;       // bit q: expert 4 lane + q has a short tile (nt of them)
  int total_main;  // tiles that are not short
  int total;       // all tiles
  int tiles[4];    // this lane's experts' tiles that are not short
};

__device__ __forceinline__ int lane_inclusive_sum(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

__device__ __forceinline__ TileScan tile_scan(const int32_t* __restrict__ offsets, int E, int BM,
                                              int nt) {
  const int lane = lane_id();
  TileScan sc;
  int mine = 0;
  sc.sbits = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * lane + q;
    const int n = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    const int rem = n % BM;
    const int sh = (rem != 0 && rem <= kShortRows) ? 1 : 0;
    sc.tiles[q] = ((n + BM - 1) / BM - sh) * nt;
    sc.sbits |= sh << q;
    mine += sc.tiles[q];
  }
  const int smine = __builtin_popcount(sc.sbits) * nt;
  sc.incl = lane_inclusive_sum(mine);
  sc.excl = sc.incl - mine;
  const int sincl = lane_inclusive_sum(smine);
  sc.sexcl = sincl - smine;
  sc.total_main = __shfl(sc.incl, kWave - 1);
  sc.total = sc.total_main + __shfl(sincl, kWave - 1);
  return sc;
}

// A wave's scan kept in LDS between units (so that it holds no registers across a unit):
// field f of lane l at words[f * 64 + l].
constexpr int kScanWords = 8 * 64;
__device__ __forceinline__ void scan_store(const TileScan& sc, int* words) {
  const int lane = lane_id();
  const int v[8] = {sc.excl, sc.incl, sc.sexcl, sc.sbits,
                    sc.tiles[0], sc.tiles[1], sc.tiles[2], sc.tiles[3]};
#pragma unroll
  for (int f = 0; f < 8; ++f) words[f * kWave + lane] = v[f];
}
__device__ __forceinline__ TileScan scan_load(const int* words, int total_main, int total) {
  const int lane = lane_id();
  TileScan sc;
  sc.excl = words[0 * kWave + lane];
  sc.incl = words[1 * kWave + lane];
  sc.sexcl = words[2 * kWave + lane];
  sc.sbits = words[3 * kWave + lane];
#pragma unroll
  for (int q = 0; q < 4; ++q) sc.tiles[q] = words[(4 + q) * kWave + lane];
  sc.total_main = total_main;
  sc.total = total;
  return sc;
}

__device__ __forceinline__ void tile_of(const TileScan& sc, const int32_t* __restrict__ offsets,
                                        int BM, int nt, int mb, int nb, bool short_last, int L,
                                        int& e_out, int& row0, int& rows, int& n_tile) {
  const int lane = lane_id();
  const int nsh = __builtin_popcount(sc.sbits) * nt;  // this lane's experts' short tiles
  const bool main_run = !short_last || L < sc.total_main;
  const int Lr = main_run ? L : L - sc.total_main;  // position in its run
  const int ex = !short_last ? sc.excl + sc.sexcl : main_run ? sc.excl : sc.sexcl;
  const int in = !short_last ? sc.incl + sc.sexcl + nsh : main_run ? sc.incl : sc.sexcl + nsh;
  const unsigned long long own = __ballot(Lr >= ex && Lr < in);
  const int owner = __ffsll((long long)own) - 1;
  int e = -1, local = 0;
  int run = ex;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int sq = ((sc.sbits >> q) & 1) * nt;
    const int cnt_q = !short_last ? sc.tiles[q] + sq : main_run ? sc.tiles[q] : sq;
    if (e < 0 && Lr < run + cnt_q) {
      e = 4 * lane + q;
      local = Lr - run;
    }
    run += cnt_q;
  }
  e = __shfl(e, owner);
  local = __shfl(local, owner);
  const int cnt = offsets[e + 1] - offsets[e];
  const int rem = cnt % BM;
  const int sh = (short_last && rem != 0 && rem <= kShortRows) ? 1 : 0;
  const int tm = (cnt + BM - 1) / BM - sh;  // this expert's M-tiles in the first run
  int m;
  if (main_run) {
    const int mbe = min(mb, tm);           // (so mbe * nt <= tm * nt, the expert's tiles)
    const int mblk = local / (mbe * nt);   // every M-block but the last has mbe M-tiles
    const int mj = min(mbe, tm - mblk * mbe);
    const int rem_l = local - mblk * mbe * nt;
    const int blk = rem_l / (mj * nb);
    const int within = rem_l - blk * mj * nb;
    m = mblk * mbe + within % mj;
    n_tile = blk * nb + within / mj;
  } else {  // the expert's last M-tile, column tile `local`
    m = tm;
    n_tile = local;
  }
  e_out = e;
  row0 = offsets[e] + m * BM;
  rows = min(BM, cnt - m * BM);
}

}  // namespace moe

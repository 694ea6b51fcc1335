// Fused bf16 routing: router logits, row softmax, top-k, gates, the Switch loss and the
// per-expert counts in one pass over x (ML Grind "Mixture-of-Experts (MoE) Routing",
// Algorithm steps 1 and 2 and the load-balancing step; ties go to the lower expert index,
// "Edge cases and conventions"), plus the dispatch ranks and row offsets that follow from the
// counts (Algorithm step 3 and Follow-up; capacity with the first routed tokens kept, as in
// "Mixture of Experts: the Sparsely-Gated Layer", "Switch: top-1, one loss, and a rate limit").
//
// Three launches:
//  1. prep (one block per 64 router rows): the router transposed to (E, D), so that both the
//     MFMA operand and the exact dot products read an expert's weights K-contiguous; for each
//     64-row block b, m_b = max_e ||W[64b .. 64b+63, e]||_2 rounded up; the routing counters
//     cleared.
//  2. route (one 256-thread block per TT tokens, TT chosen so the token tile fills at most
//     64 KB of LDS and two blocks share a CU):
//     a. the block's token tile goes from HBM into LDS once (global_load_lds_dwordx4; the
//        16-byte chunk c of row r is stored at chunk c ^ (r % 16), so the 16 rows an MFMA
//        operand read touches fall in distinct banks);
//     b. logits: v_mfma_f32_16x16x32_bf16 over the tile and the transposed router; every MFMA
//        sums 32 exact bf16 products from a zero accumulator and is folded into float64 at
//        once;
//     c. one wave per token: a rigorous bound B_t on |logit - exact logit| (every 32-term
//        float32 sum is within 32 * 2^-23 of the sum of its |products|, which Cauchy-Schwarz
//        bounds by ||x_chunk|| ||w_chunk||; over each 64-row block by ||x_t,b|| m_b), then the
//        top k + 1 by descending logit. When every gap in that sequence exceeds 2 B_t the
//        order is the exact logits' order; the k chosen logits are then recomputed exactly
//        (float64 sums of exact products, read from the LDS tile) and the gates come from
//        them. Otherwise all E logits are recomputed exactly and the top-k is taken on them;
//     d. per-block sums of the probabilities (fixed order, then rounded to multiples of 2^-40
//        and added as 64-bit integers, so the totals do not depend on block order) and counts
//        go to global counters; the last block to finish (a ticket) forms aux = E sum_e f_e P_e,
//        the counts, the row offsets (kept_e = min(count_e, capacity)) and, per group of 256
//        tokens and expert, the number of earlier routed slots (the rank base of the group).
//  3. place (one block per group of 256 tokens): each slot's rank among the group's earlier
//     slots of its expert (64-bit lane masks in LDS and popcounts), plus the group's rank base:
//     kept iff rank < capacity, row = offsets[e] + rank, perm[row] = slot, slot_row[slot] = row
//     or -1.
// Everything is deterministic: no floating-point atomics, fixed summation orders.
#include <float.h>
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "route_util.hpp"

namespace moe {
namespace {

constexpr int kFT = 256;  // threads of a routing block: 4 waves, two blocks a CU
constexpr int kFW = kFT / kWave;
constexpr int kPrepRows = 64;                    // router rows per prep block (and per bound block)
constexpr int kGroup = kDispatchTokensPerBlock;  // tokens per dispatch group
// Threads of a placement block: all of them add up the routing slots, the first kGroup (one
// per token of the group) then place the group's slots.
constexpr int kPlaceThreads = 1024;
constexpr double kPScale = 1099511627776.0;      // 2^40, the probability sums' fixed point
constexpr int kCountShift = 55;                  // the counts' place in a group slot
constexpr int kMaxTT = 256;
constexpr size_t kMaxLds = 160 * 1024;
constexpr size_t kStaticLds = 1024;  // headroom for the routing kernel's own __shared__ words
constexpr int kMaxExpertsExact = 64;  // the exact route's limit on E

typedef __attribute__((address_space(3))) const char lds_cchar_t;

__device__ __forceinline__ uint32_t lds_u32addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
// 16 bytes per lane from `src` to LDS byte address lds + 16 * lane (lds wave-uniform).
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void wait_all_vm() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  return *(lds_u32x4*)(uintptr_t)addr;
}

// Sum over the 8 lanes of each aligned group of 8 (xor 1, 2, 4); every lane of the group ends
// with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float group8_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_f32<0x141>(v);  // row_half_mirror: the other quad of the group of 8
  return v;
}
// Sum over the wave, the same value in every lane: the rows of 16 by DPP, then the 4 rows.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = group8_sum(v);
  v += dpp_f32<0x140>(v);  // row_mirror: the other group of 8 of the row
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Float64 dot products of token row `xrow` of the LDS tile (chunk swizzle `sw`) with n rows of
// the transposed router, CG rows per pass (row row_of(j) for the j-th product): lane l takes
// the 16-byte chunks c = l (mod 64), NB of them per round, and every router load of a round
// (NB x CG, 16 bytes each) is issued before any is used, so a round costs one memory latency.
// Every product of two bf16 values is exact in float64, so each sum carries float64 rounding
// only; the lane sums are added by a fixed butterfly, so the value of a product does not
// depend on which others share its pass. put(j, v) receives the wave-uniform j-th sum.
template <int CG, class RowOf, class Put>
__device__ __forceinline__ void tile_dots_f64(uint32_t xrow, int sw, const uint16_t* __restrict__ wt,
                                              int64_t D, int n, RowOf row_of, Put put) {
  constexpr int NB = 32 / CG;  // chunks per lane and round: 32 loads in flight
  const int lane = lane_id();
  const int nch = (int)(D / 8);
  for (int j0 = 0; j0 < n; j0 += CG) {
    const int nj = min(CG, n - j0);
    const uint4* wr[CG];
#pragma unroll
    for (int jj = 0; jj < CG; ++jj)
      wr[jj] = (const uint4*)(wt + (int64_t)row_of(j0 + (jj < nj ? jj : 0)) * D);
    double acc[CG];
#pragma unroll
    for (int jj = 0; jj < CG; ++jj) acc[jj] = 0.0;
    for (int c0 = 0; c0 < nch; c0 += NB * kWave) {
      uint4 wv[NB][CG];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int c = c0 + b * kWave + lane;
#pragma unroll
        for (int jj = 0; jj < CG; ++jj)  // rows past nj repeat row j0 (not used)
          wv[b][jj] = c < nch ? wr[jj][c] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int c = c0 + b * kWave + lane;
        if (c0 + b * kWave >= nch) break;
        u32x4 xv = {0u, 0u, 0u, 0u};
        if (c < nch) xv = lds_read16(xrow + 16u * (uint32_t)(c ^ sw));
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
        double xd[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xd[2 * q] = (double)__uint_as_float(xw[q] << 16);
          xd[2 * q + 1] = (double)__uint_as_float(xw[q] & 0xffff0000u);
        }
#pragma unroll
        for (int jj = 0; jj < CG; ++jj) {
          const uint32_t ww[4] = {wv[b][jj].x, wv[b][jj].y, wv[b][jj].z, wv[b][jj].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[jj] = fma(xd[2 * q], (double)__uint_as_float(ww[q] << 16), acc[jj]);
            acc[jj] = fma(xd[2 * q + 1], (double)__uint_as_float(ww[q] & 0xffff0000u), acc[jj]);
          }
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < CG; ++jj) {
      if (jj >= nj) break;
      put(j0 + jj, wave_sum(acc[jj]));
    }
  }
}

template <class RowOf, class Put>
__device__ __forceinline__ void tile_dots_any(int cg, uint32_t xrow, int sw,
                                              const uint16_t* __restrict__ wt, int64_t D, int n,
                                              RowOf row_of, Put put) {
  if (cg <= 2)
    tile_dots_f64<2>(xrow, sw, wt, D, n, row_of, put);
  else if (cg <= 4)
    tile_dots_f64<4>(xrow, sw, wt, D, n, row_of, put);
  else if (cg <= 6)
    tile_dots_f64<6>(xrow, sw, wt, D, n, row_of, put);
  else
    tile_dots_f64<8>(xrow, sw, wt, D, n, row_of, put);
}

// ---- prep ----------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void route_prep_fused_kernel(int64_t D, int E,
                                                               const uint16_t* __restrict__ w,
                                                               uint16_t* __restrict__ wt,
                                                               float* __restrict__ mb,
                                                               int32_t* __restrict__ zero,
                                                               int64_t nzero) {
  __shared__ uint16_t s_w[kPrepRows * kMaxExperts];
  __shared__ double s_n[kMaxExperts];
  const int tid = threadIdx.x;
  for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < nzero; i += (int64_t)gridDim.x * 256)
    zero[i] = 0;
  const int64_t d0 = (int64_t)blockIdx.x * kPrepRows;
  const int rows = (int)min<int64_t>(kPrepRows, D - d0);
  const uint16_t* src = w + d0 * E;  // rows d0 .. d0 + rows - 1 are contiguous
  for (int i = tid; i < rows * E; i += 256) s_w[i] = src[i];
  __syncthreads();
  for (int i = tid; i < E * kPrepRows; i += 256) {
    const int e = i / kPrepRows, dd = i % kPrepRows;
    if (dd < rows) wt[(int64_t)e * D + d0 + dd] = s_w[dd * E + e];
  }
  if (tid < E) {
    double acc = 0.0;
    for (int dd = 0; dd < rows; ++dd) {
      const double f = (double)bf16_to_f32(s_w[dd * E + tid]);
      acc = fma(f, f, acc);
    }
    s_n[tid] = acc;
  }
  __syncthreads();
  if (tid == 0) {
    double m = 0.0;
    for (int e = 0; e < E; ++e) m = fmax(m, s_n[e]);
    // an upper bound on sqrt(m), as a float
    const double up = sqrt(m) * (1.0 + 0x1p-40);
    float f = (float)up;
    if ((double)f < up) f = nextafterf(f, INFINITY);
    mb[blockIdx.x] = f;
  }
}

// ---- route ---------------------------------------------------------------------------------

struct FusedArgs {
  int64_t T, D;
  int E, k, TT, MT, NT, ksf;
  const uint16_t* x;
  const uint16_t* wt;
  const float* mb;
  const float* bias;
  int32_t* idx;
  float* gates;
  float* logits_out;        // nullable
  int32_t* nflag;           // tokens recomputed in float64 (a counter)
  unsigned long long* gslot;  // (nG, E): count << kCountShift plus the 2^-40 probability sum
};

template <int PPW, int EPL>
// (two blocks share a CU: at least 2 waves per SIMD, at most 256 VGPRs each)
__global__ __launch_bounds__(kFT, 2) void route_fused_kernel(FusedArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());
  const int TT = a.TT, E = a.E, k = a.k;
  const int64_t D = a.D, T = a.T;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int nvalid = (int)min<int64_t>(TT, T - t0);
  const uint32_t row_bytes = (uint32_t)(2 * D);
  const uint32_t lds_x = lds_u32addr(smem);
  double* region = (double*)(smem + (size_t)TT * row_bytes);
  const int nch = (int)(D / 8);     // 16-byte chunks per row
  const int nseg = (nch + 63) / 64;  // 1 KB segments per row
  const int nIc = (nch + kWave - 1) / kWave;

  // b0. the MFMA operands of the router: wave w takes tile pairs pbase + j * pstep and
  //     k-steps ks = w % ksf (mod ksf), the operands of kB of them loaded together
  const int P = a.MT * a.NT, ksf = a.ksf;
  const int pbase = wv / ksf, pstep = kFW / ksf;
  const int nks = (int)(D / 32);
  constexpr int kB = PPW == 1 ? 32 : 16 / PPW;  // k-steps whose router operands load together
  uint32_t arow[PPW];
  int asw[PPW];
  const uint16_t* bptr[PPW];
  bool pv[PPW];
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    const int p = pbase + j * pstep;
    pv[j] = p < P;
    const int m = pv[j] ? p / a.NT : 0, n = pv[j] ? p % a.NT : 0;
    int r = m * 16 + (lane & 15);
    if (r >= TT) r &= TT - 1;  // TT < 16: rows repeat (their results are not used)
    arow[j] = lds_x + (uint32_t)r * row_bytes;
    asw[j] = r & 15;
    const int e = n * 16 + (lane & 15);  // columns past E load nothing (their logits are unused)
    bptr[j] = e < E ? a.wt + (int64_t)e * D + 8 * (lane >> 4) : nullptr;
  }
  bf16x8 bv[kB][PPW];
  auto load_b = [&](int ks0) {
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int ks = min(ks0 + u * ksf, nks - 1);
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        bv[u][j] = bf16x8{};
        if (bptr[j]) bv[u][j] = *(const bf16x8*)(bptr[j] + (int64_t)ks * 32);
      }
    }
  };

  // a. the token tile, straight into LDS
  for (int i = wv; i < TT * nseg; i += kFW) {
    const int r = i / nseg, sg = i % nseg;
    if (r >= nvalid) break;
    const int pos = sg * 64 + lane;
    if (pos < nch) {
      const int c = sg * 64 + (lane ^ (r & 15));
      const uint32_t dst =
          __builtin_amdgcn_readfirstlane(lds_x + (uint32_t)r * row_bytes + (uint32_t)sg * 1024u);
      lds_dma16(a.x + (t0 + r) * D + 8 * (int64_t)c, dst);
    }
  }
  load_b(wv % ksf);  // (completes after the tile: memory operations finish in issue order)
  // the 64-row blocks' router norm bounds (D <= 8192: at most 128 of them), and the biases
  __shared__ float s_mb[128];
  __shared__ float s_bias[kMaxExperts];
  __shared__ double s_mnorm;
  for (int i = tid; i < (nch + 7) / 8; i += kFT) s_mb[i] = a.mb[i];
  for (int i = tid; i < E; i += kFT) s_bias[i] = a.bias ? a.bias[i] : 0.f;
  wait_all_vm();
  __syncthreads();
  if (wv == 0) {
    // ||m|| = sqrt(sum_b m_b^2), an upper bound (float64 sum of float32 squares, then inflated)
    double m2 = 0.0;
    for (int b = lane; b < (nch + 7) / 8; b += kWave) m2 = fma((double)s_mb[b], (double)s_mb[b], m2);
    m2 = wave_sum(m2);
    if (lane == 0) s_mnorm = sqrt(m2) * (1.0 + 0x1p-40);
  }

  // b. logits: every MFMA sums 32 products from zero; the results of kF consecutive steps are
  //    added in float32 (kF - 1 more roundings of at most 2^-24 of their running sum) and that
  //    sum is folded into float64
  constexpr int kF = kB < 8 ? kB : 8;
  double acc[PPW][4];
#pragma unroll
  for (int j = 0; j < PPW; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[j][v] = 0.0;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 part[PPW];  // the float32 sum of the current group of kF steps
  static_assert(kB % kF == 0, "fold groups within a batch");
  // a step past the end (the last batch's tail) multiplies zero operands, so every batch runs
  // all kB steps: the operand reads and the MFMAs of groups of 4 steps are issued together
  // before their results are folded
  for (int ks0 = wv % ksf; ks0 < nks; ks0 += kB * ksf) {
    if (ks0 != wv % ksf) load_b(ks0);
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (ks0 + u * ksf >= nks)
#pragma unroll
        for (int j = 0; j < PPW; ++j) bv[u][j] = bf16x8{};
    constexpr int kG = 4 / PPW;  // steps whose MFMAs are issued together
#pragma unroll
    for (int u0 = 0; u0 < kB; u0 += kG) {
      bf16x8 av[kG][PPW];
#pragma unroll
      for (int u = u0; u < u0 + kG; ++u) {
        const int c = min(ks0 + u * ksf, nks - 1) * 4 + (lane >> 4);
#pragma unroll
        for (int j = 0; j < PPW; ++j)
          av[u - u0][j] =
              __builtin_bit_cast(bf16x8, lds_read16(arow[j] + 16u * (uint32_t)(c ^ asw[j])));
      }
      f32x4 cc[kG][PPW];
#pragma unroll
      for (int u = 0; u < kG; ++u)
#pragma unroll
        for (int j = 0; j < PPW; ++j)
          cc[u][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][j], bv[u0 + u][j], zero4, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < kG; ++u)
#pragma unroll
        for (int j = 0; j < PPW; ++j) {
          if ((u0 + u) % kF == 0)
            part[j] = cc[u][j];
          else
#pragma unroll
            for (int v = 0; v < 4; ++v) part[j][v] += cc[u][j][v];
          if ((u0 + u) % kF == kF - 1)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[j][v] += (double)part[j][v];
        }
    }
  }
  // partial logits (ksf x TT x E, float64) into the region; C layout: lane l holds column
  // l % 16 and rows 4 (l / 16) + v of its tile
  {
    const int slot = wv % ksf;
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      if (!pv[j]) continue;
      const int p = pbase + j * pstep, m = p / a.NT, n = p % a.NT;
      const int col = n * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m * 16 + 4 * (lane >> 4) + v;
        if (row < TT && col < E) region[((int64_t)slot * TT + row) * E + col] = acc[j][v];
      }
    }
  }
  __syncthreads();

  // c. the tokens, one wave each (the wave's tokens are r = wv, wv + 4, ...): logits, bound,
  //    top k + 1; when the bound certifies the order, the k chosen logits exactly (gates need
  //    them to ~1e-7; with k = 1 the gate is 1 whatever the logit), else every logit exactly
  //    and the decision from them; then probabilities, gates and counts.
  double psum[EPL];
  int cnt[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    psum[i] = 0.0;
    cnt[i] = 0;
  }
  int nflag = 0;
  // every 32-term MFMA sum is within 31 * 2^-23 of the sum of its |products| (any order, either
  // rounding), the float32 additions of a fold group add at most 7 * 2^-24, the float64 folds far
  // less
  const double gamma = 35.0 * 0x1p-23;
  for (int r = wv; r < nvalid; r += kFW) {
    const int64_t t = t0 + r;
    double lg[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + kWave * i;
      lg[i] = 0.0;
      if (e < E) {
        for (int s = 0; s < ksf; ++s) lg[i] += region[(s * TT + r) * E + e];
        lg[i] += (double)s_bias[e];
      }
    }
    const uint32_t xrow = lds_x + (uint32_t)r * row_bytes;
    const int sw = r & 15;
    // ||x_t||^2 by dot2 of bf16 pairs (float32; inflated to cover its roundings). By
    // Cauchy-Schwarz over the 64-row blocks, sum_b ||x_t,b|| m_b <= ||x_t|| ||m||.
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    float xs = 0.f;
    for (int i0 = 0; i0 < nIc; i0 += 4) {
      u32x4 xv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = lane + kWave * (i0 + u);
        xv[u] = u32x4{0u, 0u, 0u, 0u};
        if (c < nch) xv[u] = lds_read16(xrow + 16u * (uint32_t)(c ^ sw));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const bf16x2_t v2 = __builtin_bit_cast(bf16x2_t, xw[h]);
          xs = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, xs, false);
        }
      }
    }
    const double xn2 = (double)wave_sum_f32(xs) * (1.0 + (double)D * 0x1p-20) + 1e-300;
    const double bx = sqrt(xn2) * s_mnorm * (1.0 + 0x1p-30);
    double lmax = 0.0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i < E) lmax = fmax(lmax, fabs(lg[i]));
    lmax = wave_max(lmax);
    const double B = gamma * bx + lmax * 0x1p-50 + 1e-30;
    double my_v[EPL];
    int my_e[EPL];
    bool sel[EPL];
    const double gap = topk_rounds_keys<EPL>(E, k, lg, sel, my_v, my_e);
    const bool flagged = !(gap > 2.0 * B + lmax * 0x1p-22);
    if (flagged) {
      // every logit exactly, and the decision from them
      tile_dots_any(8, xrow, sw, a.wt, D, E, [](int j) { return j; }, [&](int j, double v) {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (j == lane + kWave * i) lg[i] = v;
      });
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        lg[i] = lane + kWave * i < E ? lg[i] + (double)s_bias[lane + kWave * i] : 0.0;
      topk_rounds<EPL>(E, k, lg, sel, my_v, my_e, false);
      ++nflag;
    } else if (k > 1) {
      // the k chosen logits exactly (the order is already the exact one)
      auto row_of = [&](int j) {
        int e = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if ((j >> 6) == i) e = __builtin_amdgcn_readlane(my_e[i], j & 63);
        return e;
      };
      tile_dots_any(k, xrow, sw, a.wt, D, k, row_of, [&](int j, double v) {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (j == lane + kWave * i) my_v[i] = v + (double)s_bias[my_e[i]];
      });
    }
    write_logits<EPL>(a.logits_out, t, E, lg);
    double prob[EPL];
    finish_token<EPL>(E, k, t, lg, my_v, my_e, prob, a.idx, a.gates, true);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      psum[i] += prob[i];
      cnt[i] += sel[i] ? 1 : 0;
    }
  }

  // d. block sums (waves in order), added to the token group's slots as one 64-bit integer
  //    per expert: the count above kCountShift, the probability sum in units of 2^-40 below
  //    (a group's sums stay below 2^48, its counts below 2^9), so the totals do not depend on
  //    the order the blocks add them in
  __syncthreads();  // the region's partial logits are no longer read
  double* s_ps = region;                         // [kFW][E]
  int32_t* s_cn = (int32_t*)(region + kFW * E);  // [kFW][E]
  __shared__ int s_nf[kFW];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    if (e < E) {
      s_ps[wv * E + e] = psum[i];
      s_cn[wv * E + e] = cnt[i];
    }
  }
  if (lane == 0) s_nf[wv] = nflag;
  __syncthreads();
  const int64_t g = t0 / kGroup;
  for (int e = tid; e < E; e += kFT) {
    double ps = 0.0;
    int c = 0;
#pragma unroll
    for (int q = 0; q < kFW; ++q) {
      ps += s_ps[q * E + e];
      c += s_cn[q * E + e];
    }
    const unsigned long long v =
        ((unsigned long long)c << kCountShift) + (unsigned long long)llrint(ps * kPScale);
    if (v) atomicAdd(a.gslot + g * E + e, v);
  }
  if (tid == 0) {
    int nf = 0;
#pragma unroll
    for (int q = 0; q < kFW; ++q) nf += s_nf[q];
    if (nf) atomicAdd(a.nflag, nf);
  }
}

// ---- exact route (E <= 64) ------------------------------------------------------------------

// Every logit exactly: the float64 matrix cores (v_mfma_f64_16x16x4f64) sum the products of the
// bf16 inputs, each exact in float64, with float64 rounding only; nothing is left to certify.
// One block per TT = 16 MT tokens (MT M-tiles of 16 rows), Wv waves: wave w takes M-tile
// w / KP and the K-chunks c = w % KP (mod KP), KP = Wv / MT, where a chunk is 32 of D and its
// step j (0..7) gives lane group g (lane / 16) the column d = 32 c + 8 g + j, so a lane's A
// values for a chunk are 8 consecutive bf16 of its token row (one 16-byte load) and its B
// values the router entries W[d][16 n + lane % 16] of those 8 rows (E-strided, from L2).
constexpr int kXT = 16;  // tokens per M-tile: the float64 MFMA's 16 rows
constexpr int kMaxKP = 16;  // K-parts of an M-tile at most (waves a block / M-tiles)

struct ExactArgs {
  int64_t T, D;
  int E, k, MT, KP;
  int Ec;  // router columns computed: E, or 2 E with the noise router's E columns after them
  bool renorm;
  const uint16_t* x;
  const uint16_t* w;
  const uint16_t* wn;  // nullable: the noise router (D, E)
  const float* noise;  // with wn: the standard-normal draw (T, E)
  const float* bias;
  int32_t* idx;
  float* gates;
  float* logits_out;          // nullable
  unsigned long long* bslot;  // (blocks, E): count << kCountShift plus the 2^-40 probability sum
  unsigned long long* islot;  // nullable: (blocks, E), the block's final gates summed per expert
                              // in units of 2^-40 (for the importance loss)
};

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double bf16_lo_f64(uint32_t u) { return (double)__uint_as_float(u << 16); }
__device__ __forceinline__ double bf16_hi_f64(uint32_t u) {
  return (double)__uint_as_float(u & 0xffff0000u);
}

// Reductions over a row of 16 lanes (lane ^ 1, lane ^ 2, the mirrored lane of the half row, of
// the row): every lane of the row ends with the same value, in a fixed order.
__device__ __forceinline__ double row_sum16(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  return v;
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(double& bv, int& be) {
  const double ov = dpp_f64<CTRL>(bv);
  const int oe = __builtin_amdgcn_mov_dpp(be, CTRL, 0xf, 0xf, true);
  if (ov > bv || (ov == bv && oe < be)) {
    bv = ov;
    be = oe;
  }
}
// The larger logit, equal logits to the smaller expert index (a total order, so every lane of
// the row ends with the same pair).
__device__ __forceinline__ void row_argmax16(double& bv, int& be) {
  argmax_step<0xB1>(bv, be);
  argmax_step<0x4E>(bv, be);
  argmax_step<0x141>(bv, be);
  argmax_step<0x140>(bv, be);
}

// The chunk ring of a wave: slot = the chunk's A tile (16 token rows x 32 of D, 1 KB, lane l's
// MFMA operand at byte 16 l) then NT router tiles (32 rows of D x 16 experts, 32 bytes a row).
// Both arrive by global_load_lds_dwordx4, which no register waits for: the waits are explicit.
// A chunk is 64 of D: two halves h of 32. Its A tile (16 token rows x 128 bytes, 2 KB) arrives
// by two DMAs in which lanes 8 a .. 8 a + 7 fetch one row's 128 contiguous bytes (whole cache
// lines); 16-byte segment s of row r lands in slot 8 r + (s ^ (r % 8)), so the 16 rows an A
// operand read touches fall in distinct banks. The router tiles follow: with 8 experts one DMA
// of the chunk's 64 rows x 16 bytes, else per expert tile n and half h 32 rows x 16 experts
// (32 bytes a row, 1 KB).
template <int NT, bool E8>
constexpr int exact_ring() {  // chunks in flight per wave
  return E8 ? 3 : 2;
}
template <int NT, bool E8>
constexpr uint32_t exact_slot() {
  return 2048u + (E8 ? 1024u : 2048u * NT);
}
template <int NT, bool E8>
constexpr int exact_dmas() {  // loads a chunk takes
  return 2 + (E8 ? 1 : 2 * NT);
}

template <int NT, bool E8>
__device__ __forceinline__ void exact_issue(const char* const (&asrc)[2],
                                            const char* const (&bsrc)[NT], int64_t c,
                                            int64_t brow_bytes, uint32_t slot) {
  lds_dma16(asrc[0] + c * 128, slot);
  lds_dma16(asrc[1] + c * 128, slot + 1024u);
  if (E8) {
    lds_dma16(bsrc[0] + c * brow_bytes, slot + 2048u);
  } else {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        lds_dma16(bsrc[n] + c * brow_bytes + h * (brow_bytes / 2), slot + 2048u + 1024u * (2 * n + h));
  }
}

// s_waitcnt vmcnt(after * L): the loads of the `after` chunks issued after this one may stay
// in flight (vector memory operations complete in issue order); expcnt and lgkmcnt at their
// maxima, so not waited for
template <int L, int A>
__device__ __forceinline__ void exact_wait_n() {
  constexpr int n = L * A;
  static_assert(n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0xF70);
}
template <int L, int R>
__device__ __forceinline__ void exact_wait(int after) {
  switch (after) {
    case 0: exact_wait_n<L, 0>(); break;
    case 1: exact_wait_n<L, 1>(); break;
    default: if constexpr (R > 2) exact_wait_n<L, 2>(); break;
  }
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

template <int NT>
constexpr int exact_waves() {
  return NT == 1 ? 16 : NT == 2 ? 8 : 4;
}

// E8: exactly 8 experts. The products then run on v_mfma_f64_4x4x4f64 (four blocks of 4 tokens
// x 4 experts x 4 of K, two a k-step for the two expert quads), which wastes no columns where
// the 16 x 16 instruction would leave half of its 16 expert columns empty.
template <int NT, bool E8 = false>
__global__ __launch_bounds__(exact_waves<NT>() * kWave) void route_exact_kernel(ExactArgs a) {
  static_assert(!E8 || NT == 1, "8 experts are one expert tile");
  constexpr int Wv = exact_waves<NT>();
  // dynamic LDS: the waves' chunk rings, then (after the chunk loop) the partial logits of
  // every wave (Wv x NT tiles of 16 x 16, float64: 32 KB), then the probability sums and counts
  extern __shared__ __align__(16) char smem[];
  double* s_part = (double*)smem;
  const int tid = threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const int KP = a.KP, E = a.E, k = a.k;
  const int64_t D = a.D, T = a.T;
  const int TT = kXT * a.MT;
  const int64_t tb = (int64_t)blockIdx.x * TT;
  const int m = w / KP, kp = w % KP;
  const int nch = (int)(D / 64);
  const int col = lane & 15, g = lane >> 4;
  // the bias of this lane's experts (col + 16 n), loaded now so its latency is hidden
  float bias_n[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) bias_n[n] = (a.bias && 16 * n + col < E) ? a.bias[16 * n + col] : 0.f;

  // 1. partial logits. Wave w's chunks c = kp + i KP (64 of D each) go through its ring of
  //    slots: chunk i is waited for, its operands read (A by two ds_read_b128; B by single
  //    bf16 reads with 8 experts, else by two transposed reads a tile and half, which turn the
  //    expert-contiguous rows into 4 consecutive rows of one expert per lane), multiplied, and
  //    its slot refilled with the chunk a ring length later. In half h, step j gives lane
  //    group g the column d = 64 c + 32 h + 8 g + j. Rows past T repeat the last token, router
  //    columns past E repeat column 0 (neither result is used).
  {
    const int nvalid = (int)min<int64_t>(TT, T - tb);
    const char* asrc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = 8 * q + (lane >> 3), sg = (lane & 7) ^ (r & 7);
      int arow = kXT * m + r;
      if (arow >= nvalid) arow = nvalid - 1;
      asrc[q] = (const char*)(a.x + (tb + arow) * D + 8 * sg);
    }
    // the lane's A operand slots: row col, segment 4 h + g
    uint32_t aoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) aoff[h] = 16u * (uint32_t)(8 * col + ((4 * h + g) ^ (col & 7)));
    // router column c < E is W[:, c], E <= c < Ec the noise router's column c - E (both
    // matrices are D x E, so a chunk of 64 rows spans the same bytes of either)
    const char* bsrc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int cg = 16 * n + 8 * (lane & 1);
      const int64_t ro = (int64_t)(lane >> 1) * E;
      bsrc[n] = cg < E       ? (const char*)(a.w + ro + cg)
                : cg < a.Ec ? (const char*)(a.wn + ro + (cg - E))
                             : (const char*)(a.w + ro);
    }
    if (E8) bsrc[0] = (const char*)(a.w + (int64_t)lane * 8);  // row lane of the chunk's 64
    const int64_t brow_bytes = 64 * (int64_t)E * 2;  // one chunk of router rows
    constexpr int kR = exact_ring<NT, E8>();
    constexpr uint32_t kSlot = exact_slot<NT, E8>();
    constexpr int kL = exact_dmas<NT, E8>();
    const uint32_t ring = lds_u32addr(smem) + (uint32_t)w * kR * kSlot;
    const int nc = kp < nch ? (nch - kp + KP - 1) / KP : 0;
    // the wave's i-th chunk; each block starts at its own place in the row, so the blocks that
    // run at once spread their reads over the whole address range (and so over all memory
    // channels) instead of all reading the same column window of rows a fixed stride apart
    const int rot = nc > 0 ? (int)(blockIdx.x % (unsigned)nc) : 0;
    auto chunk = [&](int i) -> int64_t {
      int j = i + rot;
      if (j >= nc) j -= nc;
      return kp + (int64_t)j * KP;
    };
    f64x4 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = f64x4{0.0, 0.0, 0.0, 0.0};
    double acc8[2] = {0.0, 0.0};  // E8: the two expert quads
    for (int i = 0; i < kR && i < nc; ++i)
      exact_issue<NT, E8>(asrc, bsrc, chunk(i), brow_bytes, ring + i * kSlot);
    // the lane's transposed-read offset in a router tile: rows 8 g + (lane % 16) / 4, expert
    // columns 4 (lane % 4) .. + 3
    const uint32_t toff = (uint32_t)((8 * g + ((lane & 15) >> 2)) * 32 + 8 * (lane & 3));
    for (int i = 0; i < nc; ++i) {
      exact_wait<kL, kR>(min(kR - 1, nc - 1 - i));
      const uint32_t slot = ring + (uint32_t)(i % kR) * kSlot;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 av = lds_read16(slot + aoff[h]);
        const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
        if constexpr (E8) {
          // B lane l: expert 4 q + l % 4 of quad q, one bf16 of router row 32 h + 8 g + j
          typedef __attribute__((address_space(3))) const uint16_t lds_u16;
          const uint32_t b0 =
              slot + 2048u + (uint32_t)(32 * h + 8 * g) * 16u + 2u * (uint32_t)(lane & 3);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const double x64 = (j & 1) ? bf16_hi_f64(aw[j >> 1]) : bf16_lo_f64(aw[j >> 1]);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const uint16_t wb = *(lds_u16*)(uintptr_t)(b0 + 16u * j + 8u * q);
              acc8[q] =
                  __builtin_amdgcn_mfma_f64_4x4x4f64(x64, bf16_lo_f64(wb), acc8[q], 0, 0, 0);
            }
          }
        } else {
          v4i16_t bl[NT], bh[NT];
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const uint32_t t0 = slot + 2048u + 1024u * (2 * n + h) + toff;
            bl[n] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(uintptr_t)t0);
            bh[n] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(uintptr_t)(t0 + 128u));
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const double x64 = (j & 1) ? bf16_hi_f64(aw[j >> 1]) : bf16_lo_f64(aw[j >> 1]);
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              const short bs = j < 4 ? bl[n][j] : bh[n][j - 4];
              const double w64 = bf16_lo_f64((uint32_t)(uint16_t)bs);
              acc[n] = __builtin_amdgcn_mfma_f64_16x16x4f64(x64, w64, acc[n], 0, 0, 0);
            }
          }
        }
      }
      if (i + kR < nc) exact_issue<NT, E8>(asrc, bsrc, chunk(i + kR), brow_bytes, slot);
    }
    __syncthreads();  // every ring is drained: the partials may overwrite them
    if constexpr (E8) {
      // result layout of the 4 x 4 x 4 instruction: lane l holds token 4 ((l % 16) / 4) + l / 16,
      // expert 4 q + l % 4 (the tile's other columns are never read)
      const int tt = 4 * ((lane & 15) >> 2) + (lane >> 4);
#pragma unroll
      for (int q = 0; q < 2; ++q) s_part[(w * 16 + tt) * 16 + 4 * q + (lane & 3)] = acc8[q];
    } else {
      // result layout of the 16 x 16 x 4 instruction: lane l holds column l % 16 and rows
      // l / 16 + 4 r
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s_part[((w * NT + n) * 16 + g + 4 * r) * 16 + col] = acc[n][r];
    }
  }
  __syncthreads();

  // 2. tokens, four at a time per wave (one per row of 16 lanes; lane i of a row holds experts
  //    i + 16 n): logits (K-parts added in order, then the bias), top-k by descending logit
  //    with ties to the lower index, the row softmax, gates; choice j sits in lane j % 16 of
  //    the row, slot j / 16
  const int i = col, r = g;
  double psum[NT], gsum[NT];
  int cnt[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    psum[n] = 0.0;
    gsum[n] = 0.0;
    cnt[n] = 0;
  }
  for (int q = w; q < TT / 4; q += Wv) {
    const int tt = 4 * q + r;
    const int mm = tt / kXT, trow = tt % kXT;
    const int64_t t = tb + tt;
    const bool valid = t < T;
    double lg[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int e = 16 * n + i;
      double v = 0.0;
      if (e < a.Ec) {
        // every K-part read first (KP <= kMaxKP), then added in order
        double pv[kMaxKP];
#pragma unroll
        for (int p = 0; p < kMaxKP; ++p)
          pv[p] = p < KP ? s_part[(((mm * KP + p) * NT + n) * 16 + trow) * 16 + i] : 0.0;
#pragma unroll
        for (int p = 0; p < kMaxKP; ++p)
          if (p < KP) v += pv[p];
        if (a.bias) v += (double)bias_n[n];  // 0 past column E
      }
      lg[n] = v;
    }
    if (a.wn) {
      // noisy logits: expert e's logit plus noise[t, e] softplus(column E + e), that column
      // fetched from the lane of this row that holds it (every addend taken before any lg
      // changes; the columns past E keep their values and take no further part)
      const int64_t tc = valid ? t : T - 1;
      double add[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int e = 16 * n + i, ce = e + E;
        const int src = (lane & ~15) | (ce & 15);
        double z = 0.0;
#pragma unroll
        for (int n2 = 0; n2 < NT; ++n2) {
          const double c = __shfl(lg[n2], src);
          if ((ce >> 4) == n2) z = c;
        }
        add[n] = e < E ? (double)a.noise[tc * E + e] * (fmax(z, 0.0) + log1p(exp(-fabs(z)))) : 0.0;
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) lg[n] += add[n];
    }
    bool sel[NT];
    double my_v[NT];
    int my_e[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      sel[n] = false;
      my_v[n] = 0.0;
      my_e[n] = 0;
    }
    double v0 = 0.0;
    for (int j = 0; j < k; ++j) {
      double bv = -DBL_MAX;
      int be = INT_MAX;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int e = 16 * n + i;
        if (e < E && !sel[n] && (lg[n] > bv || (lg[n] == bv && e < be))) {
          bv = lg[n];
          be = e;
        }
      }
      row_argmax16(bv, be);
      if (j == 0) v0 = bv;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (be == 16 * n + i) sel[n] = true;
        if (j == 16 * n + i) {
          my_v[n] = bv;
          my_e[n] = be;
        }
      }
    }
    // probabilities, shifted by the largest logit (the first choice)
    double prob[NT], ex[NT];
    double ps = 0.0;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      ex[n] = (16 * n + i < E) ? exp(lg[n] - v0) : 0.0;
      ps += ex[n];
    }
    ps = row_sum16(ps);
#pragma unroll
    for (int n = 0; n < NT; ++n) prob[n] = ex[n] / ps;
    double gate[NT];
    double gs_chosen = 1.0;  // the chosen exponentials' sum (renormalised gates)
    if (a.renorm) {
      // the chosen logits' exponentials are their experts' ex values (the same exp of the same
      // difference), taken from the lanes of this row that hold them
      double gs = 0.0;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int src = (lane & ~15) | (my_e[n] & 15);
        double ev = 0.0;
#pragma unroll
        for (int n2 = 0; n2 < NT; ++n2) {
          const double c = __shfl(ex[n2], src);
          if ((my_e[n] >> 4) == n2) ev = c;
        }
        gate[n] = (16 * n + i < k) ? ev : 0.0;
        gs += gate[n];
      }
      gs = row_sum16(gs);
      gs_chosen = gs;
#pragma unroll
      for (int n = 0; n < NT; ++n) gate[n] /= gs;
    } else {
      // the chosen expert's probability, from the lane of this row that holds it
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int src = (lane & ~15) | (my_e[n] & 15);
        double pv = 0.0;
#pragma unroll
        for (int n2 = 0; n2 < NT; ++n2) {
          const double c = __shfl(prob[n2], src);
          if ((my_e[n] >> 4) == n2) pv = c;
        }
        gate[n] = pv;
      }
    }
    if (valid) {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int j = 16 * n + i;
        if (j < k) {
          a.idx[t * k + j] = my_e[n];
          a.gates[t * k + j] = (float)gate[n];
        }
        if (a.logits_out && j < E) a.logits_out[t * E + j] = (float)lg[n];
        psum[n] += prob[n];
        cnt[n] += sel[n] ? 1 : 0;
        // the lane's own expert's final gate, rounded as it is stored (its choice slot holds
        // the same quotient), for the importance sums
        if (a.islot && sel[n])
          gsum[n] += (double)(float)(a.renorm ? ex[n] / gs_chosen : prob[n]);
      }
    }
  }

  // 3. the block's probability sums and counts (the wave's four rows by two exchanges, then
  //    the waves in order), as one 64-bit integer per expert in the block's own slot (no
  //    atomics, nothing to clear beforehand)
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    psum[n] += __shfl_xor(psum[n], 16);
    psum[n] += __shfl_xor(psum[n], 32);
    cnt[n] += __shfl_xor(cnt[n], 16);
    cnt[n] += __shfl_xor(cnt[n], 32);
    gsum[n] += __shfl_xor(gsum[n], 16);
    gsum[n] += __shfl_xor(gsum[n], 32);
  }
  __syncthreads();  // the partial logits are no longer read
  double* s_ps = s_part;                        // [Wv][E]
  int32_t* s_cn = (int32_t*)(s_part + Wv * E);  // [Wv][E]
  double* s_gs = s_part + Wv * E + Wv * E / 2;  // [Wv][E] (E % 8 == 0: 8-byte aligned)
  if (r == 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int e = 16 * n + i;
      if (e < E) {
        s_ps[w * E + e] = psum[n];
        s_cn[w * E + e] = cnt[n];
        s_gs[w * E + e] = gsum[n];
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += Wv * kWave) {
    double ps = 0.0, gs = 0.0;
    int c = 0;
    for (int q = 0; q < Wv; ++q) {
      ps += s_ps[q * E + e];
      c += s_cn[q * E + e];
      gs += s_gs[q * E + e];
    }
    a.bslot[(int64_t)blockIdx.x * E + e] =
        ((unsigned long long)c << kCountShift) + (unsigned long long)llrint(ps * kPScale);
    if (a.islot) a.islot[(int64_t)blockIdx.x * E + e] = (unsigned long long)llrint(gs * kPScale);
  }
}

// ---- place ----------------------------------------------------------------------------------

struct PlaceArgs {
  int64_t T, capacity;
  int E, k, nG;
  int spg;                          // slots per group: slot s belongs to group s / spg
  int64_t nS;                       // slots
  const int32_t* idx;
  const unsigned long long* gslot;  // (nS, E), from the routing kernel
  const int32_t* nflag;             // nullable: no token was recomputed
  float* aux;
  int32_t* counts_out;   // nullable
  int32_t* uncertified;  // nullable
  int32_t* offsets;      // (E + 1); with perm null, nullable
  int32_t* perm;         // null: only the loss and the counts (one block)
  int32_t* slot_row;
  int32_t* zero;         // nullable: nzero int32 cleared by block 0 (a later kernel's counters)
  int nzero;
  const unsigned long long* islot;  // nullable: (nS, E) gate sums in units of 2^-40
  float* importance;                // with islot: the importance loss
};

// One block per group of 256 tokens, one token per thread of the first 256; the block has
// kPlaceThreads threads, so that the slot sums of step 1 take one round of loads per thread
// where there are many slots (512 routing blocks x 64 experts at T = 8192 or 16384).
//  1. From the slots (each holds a count and a probability sum of part of a group, or of a
//     whole group): each expert's total count (all groups) and rank base (the groups
//     before this one), its kept rows min(count, capacity) and the row offsets; block 0 also
//     writes the counts, the uncertified count and aux = E sum_e (count_e / (T k)) (P_e / T).
//     Every sum is over integers or in a fixed order, so the result does not depend on the
//     order of the routing blocks.
//  2. A slot's rank among the group's earlier slots of the same expert is the popcount of the
//     lower lanes' bits in its wave's 64-bit mask for that expert plus the counts of the
//     earlier waves (integer OR and popcount: order-independent); with the group's rank base
//     it is the slot's rank among all earlier tokens: kept iff rank < capacity, row =
//     offsets[e] + rank, perm[row] = slot, slot_row[slot] = row or -1.
// IMP: block 0 also adds the gate sums and forms the importance loss (a.islot non-null).
template <bool IMP>
__global__ __launch_bounds__(kPlaceThreads) void place_fused_kernel(PlaceArgs a) {
  constexpr int kW = kGroup / kWave;          // the token waves
  constexpr int kPW = kPlaceThreads / kWave;  // all waves
  static_assert(kMaxExperts <= kGroup, "one token thread per expert in the scans");
  __shared__ unsigned long long s_mask[kW][kMaxExperts];
  __shared__ int s_base[kW][kMaxExperts];
  __shared__ int s_tot[kPlaceThreads], s_gb[kPlaceThreads];
  __shared__ unsigned long long s_p[kPlaceThreads];
  __shared__ unsigned long long s_i[IMP ? kPlaceThreads : 1];  // the gate sums (block 0, IMP)
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ double s_term[kPW];
  __shared__ int s_wtot[kPW];
  const int tid = threadIdx.x, wv = wave_id(), lane = lane_id();
  const int E = a.E, k = a.k;
  const int g = blockIdx.x;
  if (g == 0 && a.zero)
    for (int i = tid; i < a.nzero; i += kPlaceThreads) a.zero[i] = 0;
  for (int i = tid; i < kW * kMaxExperts; i += kPlaceThreads) (&s_mask[0][0])[i] = 0ull;
  // this thread's token's choices, loaded now so that their latency overlaps the slots' (up to
  // 8 of them in registers; more are read again where they are used)
  constexpr int kPre = 8;
  const int64_t t = (int64_t)g * kGroup + tid;
  const bool valid = tid < kGroup && t < a.T;
  int pre[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) pre[j] = (valid && j < k) ? a.idx[t * k + j] : 0;
  auto choice = [&](int j) -> int {
    int e = 0;
#pragma unroll
    for (int q = 0; q < kPre; ++q)
      if (q == j) e = pre[q];
    return j < kPre ? e : a.idx[t * k + j];
  };
  // 1. Q threads per expert, each over the slots q, q + Q, ...: as many as one round of kC loads
  // each needs, at least kGroup / E and at most kPlaceThreads / E
  constexpr int kC = 16;  // loads in flight (more spill at 128 VGPRs, the bound of 16 waves)
  const int Q = max(1, min(kPlaceThreads / E, max(kGroup / E, (int)((a.nS + kC - 1) / kC))));
  const bool imp = IMP && g == 0;  // block 0 also adds the gate sums (importance loss)
  {
    int tot = 0, gb = 0;
    unsigned long long ps = 0, is = 0;
    if (tid < Q * E) {
      const int e = tid % E, q = tid / E;
      const int64_t gend = (int64_t)g * a.spg;  // slots of the groups before this one
      for (int64_t g0 = q; g0 < a.nS; g0 += kC * Q) {
        unsigned long long v[kC];
#pragma unroll
        for (int u = 0; u < kC; ++u) {
          const int64_t gg = g0 + (int64_t)u * Q;
          v[u] = gg < a.nS ? a.gslot[gg * E + e] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < kC; ++u) {
          const int64_t gg = g0 + (int64_t)u * Q;
          const int c = (int)(v[u] >> kCountShift);
          tot += c;
          if (gg < gend) gb += c;
          ps += v[u] & ((1ull << kCountShift) - 1ull);
        }
        if (IMP && imp) {  // block 0 only; four loads in flight keep it within 128 VGPRs
#pragma unroll 4
          for (int u = 0; u < kC; ++u) {
            const int64_t gg = g0 + (int64_t)u * Q;
            is += gg < a.nS ? a.islot[gg * E + e] : 0ull;
          }
        }
      }
    }
    s_tot[tid] = tot;
    s_gb[tid] = gb;
    s_p[tid] = ps;
    if (IMP) s_i[tid] = is;
  }
  __syncthreads();
  // the Q partial rows of each expert (row q of expert e at q E + e), summed by halving: after
  // the step of width h, entries q < h hold everything at q, q + h (any Q)
  {
    int qp = 1;
    while (qp < Q) qp *= 2;
    for (int h = qp >> 1; h >= 1; h >>= 1) {
      if (tid < h * E && tid + h * E < Q * E) {
        s_tot[tid] += s_tot[tid + h * E];
        s_gb[tid] += s_gb[tid + h * E];
        s_p[tid] += s_p[tid + h * E];
        if (IMP && imp) s_i[tid] += s_i[tid + h * E];
      }
      __syncthreads();
    }
  }
  // expert offsets: an exclusive scan of the kept counts, within each wave of 64 experts, then
  // the waves' totals (E <= kGroup)
  {
    const int kept = tid < E ? (a.capacity < 0 ? s_tot[tid]
                                               : (int)min<int64_t>((int64_t)s_tot[tid], a.capacity))
                             : 0;
    int incl = kept;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) s_wtot[wv] = incl;
    __syncthreads();
    int before = 0;
    for (int q = 0; q < wv; ++q) before += s_wtot[q];
    if (tid < E) s_off[tid] = before + incl - kept;
    if (tid == E - 1) s_off[E] = before + incl;
  }
  if (g == 0) {
    // the loss: each expert's term, summed over a wave by exchanges, then the waves in order
    double term = 0.0;
    if (tid < E) {
      if (a.counts_out) a.counts_out[tid] = s_tot[tid];
      term = ((double)s_tot[tid] / ((double)a.T * (double)k)) *
             (((double)s_p[tid] / kPScale) / (double)a.T);
    }
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) term += __shfl_xor(term, d, kWave);
    if (lane == 0) s_term[wv] = term;
    __syncthreads();
    if (tid == 0) {
      double sum = 0.0;
      for (int q = 0; q < kW; ++q) sum += s_term[q];  // waves past kW hold no expert
      *a.aux = (float)((double)E * sum);
      if (a.uncertified) *a.uncertified = a.nflag ? *a.nflag : 0;
    }
    if (IMP && imp && wv == 0) {
      // the importance loss (E <= 64: one wave): each expert's gate total (an integer sum of
      // the slots above, so in no particular order), then the squared coefficient of
      // variation of the E totals (population variance over the squared mean), by exchanges
      // in a fixed order
      const double ge = lane < E ? (double)s_i[lane] / kPScale : 0.0;
      double m = ge;
#pragma unroll
      for (int d = kWave / 2; d >= 1; d >>= 1) m += __shfl_xor(m, d, kWave);
      m /= (double)E;
      double v = lane < E ? (ge - m) * (ge - m) : 0.0;
#pragma unroll
      for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
      if (lane == 0) *a.importance = m > 0.0 ? (float)((v / (double)E) / (m * m)) : 0.f;
    }
    if (a.offsets)
      for (int e = tid; e <= E; e += kPlaceThreads) a.offsets[e] = s_off[e];
  }
  if (!a.perm) return;
  // 2. ranks within the group and placement
  if (valid)
    for (int j = 0; j < k; ++j) atomicOr(&s_mask[wv][choice(j)], 1ull << lane);
  __syncthreads();
  for (int e = tid; e < E; e += kPlaceThreads) {
    int run = s_gb[e];
#pragma unroll
    for (int q = 0; q < kW; ++q) {
      s_base[q][e] = run;
      run += __popcll(s_mask[q][e]);
    }
  }
  __syncthreads();
  if (!valid) return;
  const unsigned long long lower = (1ull << lane) - 1ull;
  for (int j = 0; j < k; ++j) {
    const int64_t sl = t * k + j;
    const int e = choice(j);
    const int rank = s_base[wv][e] + __popcll(s_mask[wv][e] & lower);
    int row = -1;
    if (a.capacity < 0 || rank < a.capacity) {
      row = s_off[e] + rank;
      a.perm[row] = (int32_t)sl;
    }
    a.slot_row[sl] = row;
  }
}

// ---- host side -----------------------------------------------------------------------------

int pow2_floor(int64_t v) {
  int p = 1;
  while ((int64_t)p * 2 <= v) p *= 2;
  return p;
}

struct FusedShape {
  int TT, MT, NT, P, ksf, ppw, epl;
  size_t region, lds;
};

FusedShape fused_shape(const Problem& p) {
  FusedShape f{};
  f.NT = (p.E + 15) / 16;
  // the token tile fills at most 64 KB of LDS (two blocks per CU); at most 16 MFMA tile pairs
  int TT = pow2_floor(std::max<int64_t>(4, 32768 / p.D));
  TT = std::min(TT, kMaxTT);
  while (TT > 4 && ((TT + 15) / 16) * f.NT > 16) TT /= 2;
  f.TT = TT;
  f.MT = (TT + 15) / 16;
  f.P = f.MT * f.NT;
  f.ksf = 1;  // waves sharing a tile pair split its k-steps
  while (f.P * f.ksf * 2 <= kFW) f.ksf *= 2;
  const int pairs_per_wave = (f.P * f.ksf + kFW - 1) / kFW;
  f.ppw = pairs_per_wave <= 1 ? 1 : pairs_per_wave <= 2 ? 2 : 4;
  f.epl = p.E <= 64 ? 1 : p.E <= 128 ? 2 : 4;
  f.region = std::max<size_t>({(size_t)f.ksf * TT * p.E * 8, (size_t)kFW * p.E * 12,
                               (size_t)kFT * 8 + kMaxExperts * 4});
  f.region = (f.region + 15) & ~size_t(15);
  f.lds = (size_t)TT * 2 * p.D + f.region;
  return f;
}

struct FusedLayout {
  size_t wt, mb, zero, nflag, gslot, bytes;
  int64_t nP, nG, nzero;
};

FusedLayout fused_layout(const Problem& p) {
  FusedLayout L{};
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off = (off + n + 255) & ~size_t(255);
    return o;
  };
  L.nP = (p.D + kPrepRows - 1) / kPrepRows;
  L.nG = (p.T + kGroup - 1) / kGroup;
  L.wt = take((size_t)p.E * p.D * 2);
  L.mb = take((size_t)L.nP * 4);
  // the counters cleared by prep, contiguous: the recomputed-token count, then the group slots
  L.zero = off;
  L.nflag = L.zero;
  L.gslot = L.zero + 8;
  const size_t end = L.gslot + (size_t)L.nG * p.E * 8;
  L.nzero = (int64_t)((end - L.zero) / 4);
  take(end - L.zero);
  L.bytes = off;
  return L;
}

// The exact route: E <= 64 experts in NT tiles of 16; the block's M-tiles grow (fewer,
// larger blocks) only past 512 blocks of one M-tile, which bounds the slots the place kernel
// reads; a group of 256 tokens is always whole blocks.
struct ExactShape {
  int NT, Wv, MT, KP, TT;
  int64_t nblk;
};

// (E % 8 == 0: a router row is whole 16-byte granules, so every granule a DMA reads lies in
// its row)
bool exact_route_shape(const Problem& p) {
  return p.dtype == MOE_BF16 && p.E >= 8 && p.E <= kMaxExpertsExact && p.E % 8 == 0 &&
         p.top_k <= p.E &&
         p.D >= 64 && p.D % 64 == 0 && p.T > 0 && p.T < ((int64_t)1 << 23);
}

// cols: the router columns computed (E, or 2 E with router noise). MT, and so the block count,
// does not depend on it (MT <= 4 <= Wv).
ExactShape exact_shape(const Problem& p, int cols = 0) {
  ExactShape f{};
  f.NT = ((cols > 0 ? cols : p.E) + 15) / 16;
  f.Wv = f.NT == 1 ? 16 : f.NT == 2 ? 8 : 4;
  f.MT = 1;
  while (f.MT < 4 && f.MT < f.Wv && (p.T + kXT * f.MT - 1) / (kXT * f.MT) > 512) f.MT *= 2;
  f.KP = f.Wv / f.MT;
  f.TT = kXT * f.MT;
  f.nblk = (p.T + f.TT - 1) / f.TT;
  return f;
}

// Dynamic LDS of the exact route: the larger of the waves' chunk rings and the partial logits.
template <int NT, bool E8>
size_t exact_lds_bytes() {
  const size_t ring = (size_t)exact_waves<NT>() * exact_ring<NT, E8>() * exact_slot<NT, E8>();
  const size_t part = (size_t)exact_waves<NT>() * NT * 256 * 8;
  return ring > part ? ring : part;
}

template <int NT, bool E8 = false>
hipError_t launch_exact_inst(const ExactShape& f, const ExactArgs& a, hipStream_t s) {
  const size_t lds = exact_lds_bytes<NT, E8>();
  // dynamic LDS past 64 KB needs the kernel's limit raised to it (once per device)
  static bool raised[64] = {};
  int dev = 0;
  if (lds > 64 * 1024) {
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!raised[dev]) {
      const hipError_t e = hipFuncSetAttribute((const void*)route_exact_kernel<NT, E8>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
      if (e != hipSuccess) return e;
      raised[dev] = true;
    }
  }
  hipLaunchKernelGGL((route_exact_kernel<NT, E8>), dim3((unsigned)f.nblk),
                     dim3((unsigned)(exact_waves<NT>() * kWave)), lds, s, a);
  return hipGetLastError();
}

// the probability-sum slots, then the gate-sum slots (the importance loss), each (blocks, E)
size_t exact_slot_bytes(const Problem& p) {
  return (((size_t)exact_shape(p).nblk * p.E * 8) + 255) & ~size_t(255);
}
size_t exact_ws_bytes(const Problem& p) { return 2 * exact_slot_bytes(p); }

template <int PPW, int EPL>
hipError_t launch_fused_inst(const FusedShape& f, const FusedArgs& a, unsigned nblk,
                             hipStream_t s) {
  // dynamic LDS past 64 KB needs the kernel's limit raised to it (once per size reached)
  static size_t lds_allowed = 64 * 1024;
  if (f.lds > lds_allowed) {
    const hipError_t e = hipFuncSetAttribute((const void*)route_fused_kernel<PPW, EPL>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)f.lds);
    if (e != hipSuccess) return e;
    lds_allowed = f.lds;
  }
  hipLaunchKernelGGL((route_fused_kernel<PPW, EPL>), dim3(nblk), dim3(kFT), f.lds, s, a);
  return hipGetLastError();
}

}  // namespace

bool fused_route_applies(const Problem& p, const RouteOpts& o, bool importance) {
  if (p.dtype != MOE_BF16) return false;
  // router noise: the noise router's E columns beside the E logit columns, 2 E <= 64
  if (o.w_noise) return exact_route_shape(p) && 2 * p.E <= kMaxExpertsExact;
  if (exact_route_shape(p)) return true;  // either gate rule, with or without importance
  if (importance) return false;
  if (!o.renorm) return false;
  if (p.T <= 0 || p.D % 128 != 0 || p.D > 8192 || p.E > kMaxExperts) return false;
  if (p.T >= (int64_t)1 << 23) return false;  // the 2^-40 probability sums stay below 2^63
  // with many choices per token the exact chosen logits (k D float64 products a token, on the
  // vector units) outweigh the pass over x that the fused path saves
  if (p.top_k > 2) return false;
  return fused_shape(p).lds + kStaticLds <= kMaxLds;
}

size_t fused_route_ws_bytes(const Problem& p) {
  return exact_route_shape(p) ? exact_ws_bytes(p) : fused_layout(p).bytes;
}

hipError_t launch_route_fused(const Problem& p, const void* x, const void* w_router,
                              const float* bias, bool renorm, int32_t* idx, float* gates,
                              float* logits_out, void* fws, hipStream_t s, bool importance,
                              const void* w_noise, const float* noise) {
  if (exact_route_shape(p)) {
    const bool nz = w_noise != nullptr;
    const ExactShape f = exact_shape(p, nz ? 2 * p.E : p.E);
    ExactArgs a{};
    a.T = p.T;
    a.D = p.D;
    a.E = p.E;
    a.k = p.top_k;
    a.MT = f.MT;
    a.KP = f.KP;
    a.renorm = renorm;
    a.Ec = nz ? 2 * p.E : p.E;
    a.x = (const uint16_t*)x;
    a.w = (const uint16_t*)w_router;
    a.wn = (const uint16_t*)w_noise;
    a.noise = nz ? noise : nullptr;
    a.bias = bias;
    a.idx = idx;
    a.gates = gates;
    a.logits_out = logits_out;
    a.bslot = (unsigned long long*)fws;
    a.islot = importance ? (unsigned long long*)((char*)fws + exact_slot_bytes(p)) : nullptr;
    switch (f.NT) {
      case 1:
        return p.E == 8 && !nz ? launch_exact_inst<1, true>(f, a, s) : launch_exact_inst<1>(f, a, s);
      case 2: return launch_exact_inst<2>(f, a, s);
      case 3: return launch_exact_inst<3>(f, a, s);
      default: return launch_exact_inst<4>(f, a, s);
    }
  }
  const FusedLayout L = fused_layout(p);
  const FusedShape f = fused_shape(p);
  char* b = (char*)fws;
  hipLaunchKernelGGL(route_prep_fused_kernel, dim3((unsigned)L.nP), dim3(256), 0, s, p.D, p.E,
                     (const uint16_t*)w_router, (uint16_t*)(b + L.wt), (float*)(b + L.mb),
                     (int32_t*)(b + L.zero), L.nzero);
  FusedArgs a{};
  a.T = p.T;
  a.D = p.D;
  a.E = p.E;
  a.k = p.top_k;
  a.TT = f.TT;
  a.MT = f.MT;
  a.NT = f.NT;
  a.ksf = f.ksf;
  a.x = (const uint16_t*)x;
  a.wt = (const uint16_t*)(b + L.wt);
  a.mb = (const float*)(b + L.mb);
  a.bias = bias;
  a.idx = idx;
  a.gates = gates;
  a.logits_out = logits_out;
  a.nflag = (int32_t*)(b + L.nflag);
  a.gslot = (unsigned long long*)(b + L.gslot);
  const unsigned nblk = (unsigned)((p.T + f.TT - 1) / f.TT);
#define MOE_FUSED(PPWV, EPLV) return launch_fused_inst<PPWV, EPLV>(f, a, nblk, s)
  if (f.epl == 1) {
    if (f.ppw == 1) MOE_FUSED(1, 1);
    if (f.ppw == 2) MOE_FUSED(2, 1);
    MOE_FUSED(4, 1);
  } else if (f.epl == 2) {
    if (f.ppw == 1) MOE_FUSED(1, 2);
    if (f.ppw == 2) MOE_FUSED(2, 2);
    MOE_FUSED(4, 2);
  } else {
    if (f.ppw == 1) MOE_FUSED(1, 4);
    if (f.ppw == 2) MOE_FUSED(2, 4);
    MOE_FUSED(4, 4);
  }
#undef MOE_FUSED
}

hipError_t launch_place_fused(const Problem& p, const int32_t* idx, const void* fws, float* aux,
                              int32_t* counts_out, int32_t* uncertified, int32_t* offsets,
                              int32_t* perm, int32_t* slot_row, hipStream_t s, int32_t* zero,
                              int nzero, float* importance) {
  const FusedLayout L = fused_layout(p);
  PlaceArgs a{};
  a.T = p.T;
  a.capacity = p.capacity;
  a.E = p.E;
  a.k = p.top_k;
  a.nG = (int)L.nG;
  a.idx = idx;
  if (exact_route_shape(p)) {  // one slot per routing block, nothing recomputed
    const ExactShape f = exact_shape(p);
    a.spg = kGroup / f.TT;
    a.nS = f.nblk;
    a.gslot = (const unsigned long long*)fws;
    a.nflag = nullptr;
    if (importance) {  // the gate sums follow the probability sums
      a.islot = (const unsigned long long*)((const char*)fws + exact_slot_bytes(p));
      a.importance = importance;
    }
  } else {
    a.spg = 1;
    a.nS = L.nG;
    a.gslot = (const unsigned long long*)((const char*)fws + L.gslot);
    a.nflag = (const int32_t*)((const char*)fws + L.nflag);
  }
  a.aux = aux;
  a.counts_out = counts_out;
  a.uncertified = uncertified;
  a.offsets = offsets;
  a.perm = perm;
  a.slot_row = slot_row;
  a.zero = zero;
  a.nzero = nzero;
  const unsigned grid = perm ? (unsigned)L.nG : 1u;
  if (a.islot)
    hipLaunchKernelGGL(place_fused_kernel<true>, dim3(grid), dim3(kPlaceThreads), 0, s, a);
  else
    hipLaunchKernelGGL(place_fused_kernel<false>, dim3(grid), dim3(kPlaceThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe

// Routing: router logits, row softmax, top-k by descending logit, gates = softmax of the
// k chosen logits, and the per-block partial sums the Switch loss needs.
// (ML Grind "Mixture-of-Experts (MoE) Routing", Algorithm steps 1 and 2 and the
// load-balancing step; ties go to the lower expert index, "Edge cases and conventions".)
//
// The selection runs one wavefront per token: lane l holds experts l, l+64, l+128, l+192
// (E <= 256), so the softmax and the top-k are wave-wide shuffles over registers.
//
// float32 layers: the logits are accumulated in float64 from exactly widened inputs (a
// product of two float32 values is exact in float64), one wave per token.
//
// bfloat16 layers (the HBM-bound path):
//  1. prep:   the router weights are transposed to (E, D) and max_e ||W[:, e]||_2 is taken.
//  2. logits: bf16 MFMA (16x16x32) over tiles of 64 tokens x all experts, the K range split
//             over blocks when there are too few token tiles to fill the chip. Every MFMA
//             sums 32 exact bf16 products into a zeroed float32 accumulator, and that
//             result is folded into float64 at once, so float32 rounding never accumulates
//             past 32 terms. Each split writes float32 partial logits and partial ||x_t||^2.
//  3. select: partials summed in float64 in split order, bias added. A rigorous bound B_t on
//             |logit - exact logit| is formed from the accumulation error of every 32-term
//             MFMA sum (Cauchy-Schwarz: <= 32 * 2^-23 * ||x_t|| * ||W_e||), the rounding of
//             the partials to float32, and the float64 sums. If two consecutive logits among
//             the k+1 largest are within 2 B_t, the decision is not certified and the token's
//             logits are recomputed in float64 from the exact products; otherwise the order of
//             the computed logits is the order of the exact ones. Either way the top-k equals
//             the one taken on exact logits. The k chosen logits are then recomputed exactly
//             (k dot products in float64) and the gates come from those; the probabilities
//             that feed the loss come from the float64-folded MFMA logits.
//
// Router options (Sparsely-Gated Layer page, "The one formula" and "The code", router()
// stages (2) and (5); "Hot shards"):
//  * noise: the decision logits are logits + noise[t, e] * softplus(x_t . W_noise[:, e]), the
//    standard-normal draw given as a (T, E) float32 input. The router product covers the 2E
//    columns [W | W_noise]; the noise columns' own error bound, propagated through softplus
//    (1-Lipschitz) and scaled by |noise|, is added to B_t before the certification test, and
//    the exact recompute of the chosen logits includes their noise terms.
//  * no renormalisation: the gates are the chosen experts' probabilities over all E experts,
//    which needs every logit of the token to the gates' accuracy, so every token takes the
//    exact float64 path of the fallback kernel.
//  * importance loss: the squared coefficient of variation of the per-expert sums of the
//    final gates, from per-block partial sums taken in token order and added in a fixed
//    order, so the result does not depend on scheduling.
#include <float.h>
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "route_util.hpp"

namespace moe {
namespace {

constexpr int kEPL = kMaxExperts / kWave;  // experts per lane
constexpr int kRouteThreads = 512;
constexpr int kRouteWaves = kRouteThreads / kWave;

// MFMA logits tiling
constexpr int kLT = 64;     // tokens per block (4 waves x 16)
constexpr int kLKB = 256;   // K per stage (LDS router chunk, A registers)
constexpr int kMinKSplit = 256;

// softplus(z) = log(1 + e^z), in float64 without overflow.
__device__ __forceinline__ double softplus_f64(double z) {
  return z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z));
}

template <typename TIn, int EPL>
__device__ __forceinline__ void logits_f64(const TIn* __restrict__ x, const TIn* __restrict__ w,
                                           int64_t t, int64_t D, int E, double lg[EPL]) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < EPL; ++i) lg[i] = 0.0;
  const TIn* xr = x + t * D;
  for (int64_t d = 0; d < D; ++d) {
    const double xv = load_as_f64(xr, d);
    const TIn* wr = w + d * E;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E) lg[i] = fma(xv, load_as_f64(wr, e), lg[i]);
    }
  }
}

// Float64 dot products of one bf16 token row with n rows of the transposed router, CG rows
// per pass over D (the row of the j-th product is row_of(j)): each lane takes the 16-byte
// slices c = lane (mod 64) of x and of the CG rows, all loads of a pass in flight at once.
// Every product of two bf16 values is exact in float64, and so is its conversion, so the
// sums carry only float64 rounding. put(j, v) receives the wave-uniform j-th sum.
template <int CG, class RowOf, class Put>
__device__ __forceinline__ void token_dots_f64(const uint16_t* __restrict__ x,
                                               const uint16_t* __restrict__ wt, int64_t t,
                                               int64_t D, int n, RowOf row_of, Put put) {
  const int lane = lane_id();
  const uint4* xr = (const uint4*)(x + t * D);
  const int64_t nc = D / 8;
  for (int j0 = 0; j0 < n; j0 += CG) {
    const int nj = min(CG, n - j0);
    const uint4* wr[CG];
#pragma unroll
    for (int jj = 0; jj < CG; ++jj)
      wr[jj] = (const uint4*)(wt + (int64_t)row_of(j0 + (jj < nj ? jj : 0)) * D);
    double acc[CG];
#pragma unroll
    for (int jj = 0; jj < CG; ++jj) acc[jj] = 0.0;
    constexpr int kUnroll = CG <= 4 ? 2 : 1;  // loads in flight vs registers
#pragma unroll kUnroll
    for (int64_t c = lane; c < nc; c += kWave) {
      const uint4 xv = xr[c];
      uint4 wv[CG];
#pragma unroll
      for (int jj = 0; jj < CG; ++jj) wv[jj] = wr[jj][c];  // duplicates of row j0 past nj
#pragma unroll
      for (int jj = 0; jj < CG; ++jj) acc[jj] += dot8_f64(xv, wv[jj]);
    }
#pragma unroll
    for (int jj = 0; jj < CG; ++jj) {
      if (jj >= nj) break;
      put(j0 + jj, wave_sum(acc[jj]));
    }
  }
}

// Exact-product float64 logits of the k chosen experts of one bf16 token (gates need the
// differences of these to ~1e-7 absolute, which a float32 partial cannot carry when the
// logits are large). CG >= k does it in one pass over D.
template <int EPL, int CG>
__device__ __forceinline__ void chosen_logits_f64(const uint16_t* __restrict__ x,
                                                  const uint16_t* __restrict__ wt,
                                                  const float* __restrict__ bias, int64_t t,
                                                  int64_t D, int k, const int my_e[EPL],
                                                  double my_v[EPL]) {
  const int lane = lane_id();
  auto row_of = [&](int j) {
    int e = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if ((j >> 6) == i) e = __shfl(my_e[i], j & 63);
    return e;
  };
  // the chosen experts' biases, loaded together (lane j holds choice j's)
  double my_b[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    my_b[i] = (bias && lane + kWave * i < k) ? (double)bias[my_e[i]] : 0.0;
  auto put = [&](int j, double v) {
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (j == lane + kWave * i) my_v[i] = v + my_b[i];
  };
  token_dots_f64<CG>(x, wt, t, D, k, row_of, put);
}


// The same with router noise: the chosen logits are x.W_e + b_e + noise[t, e] * softplus(
// x.W_noise[:, e]), both dot products exact-product float64 (2k rows of wt: the chosen
// experts' router rows, then their noise rows E + e).
template <int EPL, int CG>
__device__ __forceinline__ void chosen_logits_noisy_f64(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wt,
    const float* __restrict__ bias, const float* __restrict__ noise, int64_t t, int64_t D, int E,
    int k, const int my_e[EPL], double my_v[EPL]) {
  const int lane = lane_id();
  auto expert_of = [&](int j) {
    int e = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if ((j >> 6) == i) e = __shfl(my_e[i], j & 63);
    return e;
  };
  auto row_of = [&](int j) { return j < k ? expert_of(j) : E + expert_of(j - k); };
  double my_b[EPL], my_n[EPL], my_g[EPL], my_z[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const bool mine = lane + kWave * i < k;
    my_b[i] = (bias && mine) ? (double)bias[my_e[i]] : 0.0;
    my_n[i] = mine ? (double)noise[t * E + my_e[i]] : 0.0;
    my_g[i] = 0.0;
    my_z[i] = 0.0;
  }
  auto put = [&](int j, double v) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (j == lane + kWave * i) my_g[i] = v;
      if (j - k == lane + kWave * i) my_z[i] = v;
    }
  };
  token_dots_f64<CG>(x, wt, t, D, 2 * k, row_of, put);
#pragma unroll
  for (int i = 0; i < EPL; ++i) my_v[i] = my_g[i] + my_b[i] + my_n[i] * softplus_f64(my_z[i]);
}

// Per-block partials of sum_t probs[t, e] and of the expert counts, in fixed order.
template <int EPL>
struct BlockPartials {
  double psum[EPL];
  int cnt[EPL];
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      psum[i] = 0.0;
      cnt[i] = 0;
    }
  }
  __device__ void add(const double prob[EPL], const bool sel[EPL]) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      psum[i] += prob[i];
      cnt[i] += sel[i] ? 1 : 0;
    }
  }
};

template <int WAVES, int EPL>
__device__ __forceinline__ void write_block_partials(const BlockPartials<EPL>& bp, int E,
                                                     double* __restrict__ psum_blk,
                                                     int32_t* __restrict__ count_blk) {
  __shared__ double s_psum[WAVES][kMaxExperts];
  __shared__ int s_cnt[WAVES][kMaxExperts];
  const int wv = wave_id(), lane = lane_id();
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    s_psum[wv][lane + kWave * i] = bp.psum[i];
    s_cnt[wv][lane + kWave * i] = bp.cnt[i];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += WAVES * kWave) {
    double a = 0.0;
    int c = 0;
#pragma unroll
    for (int q = 0; q < WAVES; ++q) {
      a += s_psum[q][e];
      c += s_cnt[q][e];
    }
    // expert-major: the loss reduction then reads each expert's partials contiguously
    psum_blk[(int64_t)e * gridDim.x + blockIdx.x] = a;
    count_blk[(int64_t)e * gridDim.x + blockIdx.x] = c;
  }
}

// ---- float32 layers -----------------------------------------------------------------------

template <typename TIn, int EPL>
__global__ __launch_bounds__(kRouteThreads) void route_f64_kernel(
    int64_t T, int64_t D, int E, int k, const TIn* __restrict__ x, const TIn* __restrict__ w,
    const float* __restrict__ bias, const TIn* __restrict__ w_noise,
    const float* __restrict__ noise, bool renorm, int32_t* __restrict__ idx,
    float* __restrict__ gates,
    float* __restrict__ logits_out, double* __restrict__ psum_blk,
    int32_t* __restrict__ count_blk, int32_t* __restrict__ ticket,
    int32_t* __restrict__ uncertified) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *ticket = 0;  // the loss reduction that follows counts its blocks here
    if (uncertified) *uncertified = 0;  // float32 layers never need a recompute
  }
  BlockPartials<EPL> bp;
  bp.zero();
  const int64_t t0 = (int64_t)blockIdx.x * kRouteTokensPerBlock;
  for (int q = wave_id(); q < kRouteTokensPerBlock; q += kRouteWaves) {
    const int64_t t = t0 + q;
    if (t >= T) break;
    double lg[EPL], prob[EPL], my_v[EPL];
    int my_e[EPL];
    bool sel[EPL];
    logits_f64<TIn, EPL>(x, w, t, D, E, lg);
    add_bias<EPL>(bias, E, lg);
    if (w_noise) {
      double z[EPL];
      logits_f64<TIn, EPL>(x, w_noise, t, D, E, z);
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane_id() + kWave * i;
        if (e < E) lg[i] += (double)noise[t * E + e] * softplus_f64(z[i]);
      }
    }
    write_logits<EPL>(logits_out, t, E, lg);
    topk_rounds<EPL>(E, k, lg, sel, my_v, my_e, false);
    finish_token<EPL>(E, k, t, lg, my_v, my_e, prob, idx, gates, renorm);
    bp.add(prob, sel);
  }
  write_block_partials<kRouteWaves, EPL>(bp, E, psum_blk, count_blk);
}

// ---- bfloat16 layers ----------------------------------------------------------------------

// wt[r][d] = w[d][r] for rows r < E and w_noise[d][r - E] for rows E .. 2E - 1 (one block
// per row, gridDim.x rows); wnorm[r] = the row's ||.||_2 (float64). The sum of squares is
// reduced in a fixed order (per-thread, then an LDS tree). Also zeroes the counters that the
// later routing kernels of the call accumulate into.
__global__ __launch_bounds__(256) void router_prep_kernel(int64_t D, int E,
                                                          const uint16_t* __restrict__ w,
                                                          const uint16_t* __restrict__ w_noise,
                                                          uint16_t* __restrict__ wt,
                                                          double* __restrict__ wnorm,
                                                          int32_t* __restrict__ ticket,
                                                          int32_t* __restrict__ nlist) {
  __shared__ double s_part[256];
  const int e = blockIdx.x;
  if (e == 0 && threadIdx.x == 0) {
    *ticket = 0;
    nlist[0] = 0;
    nlist[1] = 0;
  }
  const uint16_t* src = e < E ? w : w_noise;
  const int col = e < E ? e : e - E;
  double acc = 0.0;
#pragma unroll 4
  for (int64_t d = threadIdx.x; d < D; d += 256) {
    const uint16_t v = src[d * E + col];
    wt[(int64_t)e * D + d] = v;
    const double f = (double)bf16_to_f32(v);
    acc = fma(f, f, acc);
  }
  s_part[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if ((int)threadIdx.x < h) s_part[threadIdx.x] += s_part[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) wnorm[e] = sqrt(s_part[0]);
}

template <int NT>  // tiles of 16 experts
// Partial logits of E router rows (wt, (E, D)) over one K split (blockIdx.y): columns
// col0 .. col0 + E - 1 of `part`, whose token rows are ldp floats apart. xsq (nullable)
// receives the partial ||x_t||^2.
__global__ __launch_bounds__(256) void route_logits_mfma_kernel(
    int64_t T, int64_t D, int E, int64_t kc, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ wt, float* __restrict__ part, float* __restrict__ xsq, int ldp,
    int col0) {
  __shared__ __align__(16) uint16_t sB[NT * 16][kLKB + 8];
  const int lane = lane_id(), wv = wave_id();
  const int64_t t0 = (int64_t)blockIdx.x * kLT + wv * 16;
  const int s = blockIdx.y;
  const int64_t kbeg = (int64_t)s * kc;
  const int64_t kend = min(D, kbeg + kc);
  const int64_t row = t0 + (lane & 15);
  const bool row_ok = row < T;
  const int koff = 8 * (lane >> 4);
  const uint16_t* xr = x + (row_ok ? row : 0) * D + koff;

  double acc[NT][4];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[n][v] = 0.0;
  float xs = 0.f;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  constexpr int kSteps = kLKB / 32;

  uint4 a_next[kSteps];
  auto load_a = [&](int64_t kb, uint4 (&dst)[kSteps]) {
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const int64_t kk = kb + 32 * j + koff;
      dst[j] = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok && kk < kend) dst[j] = *(const uint4*)(xr + kb + 32 * j);
    }
  };
  load_a(kbeg, a_next);
  for (int64_t kb = kbeg; kb < kend; kb += kLKB) {
    uint4 a[kSteps];
#pragma unroll
    for (int j = 0; j < kSteps; ++j) a[j] = a_next[j];
    __syncthreads();  // previous chunk's LDS reads are done
    for (int i = threadIdx.x; i < NT * 16 * (kLKB / 8); i += 256) {
      const int e = i / (kLKB / 8), q = i % (kLKB / 8);
      const int64_t kk = kb + 8 * q;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (e < E && kk < kend) v = *(const uint4*)(wt + (int64_t)e * D + kk);
      *(uint4*)&sB[e][8 * q] = v;
    }
    if (kb + kLKB < kend) load_a(kb + kLKB, a_next);  // in flight during this chunk
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, a[j]);
      const uint32_t aw[4] = {a[j].x, a[j].y, a[j].z, a[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = __uint_as_float(aw[q] << 16), hi = __uint_as_float(aw[q] & 0xffff0000u);
        xs = fmaf(lo, lo, xs);
        xs = fmaf(hi, hi, xs);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const bf16x8 bv = *(const bf16x8*)&sB[n * 16 + (lane & 15)][32 * j + koff];
        const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, zero4, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[n][v] += (double)c[v];
      }
    }
  }
  // lanes l, l^16, l^32, l^48 hold the same token row
  xs += __shfl_xor(xs, 16);
  xs += __shfl_xor(xs, 32);
  // 16x16 accumulator layout: lane l holds expert column l % 16, token rows 4*(l/16) + v
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t t = t0 + 4 * (lane >> 4) + v;
      const int e = n * 16 + (lane & 15);
      if (t < T && e < E) part[((int64_t)s * T + t) * ldp + col0 + e] = (float)acc[n][v];
    }
  if (xsq && lane < 16 && row_ok) xsq[(int64_t)s * T + row] = xs;
}

constexpr int kSelWaves = kRouteTokensPerBlock;  // one token per wave
// Up to this many experts, the select kernel recomputes a flagged token's logits itself.
constexpr int kInWaveExact = 16;

// uncertified = the listed tokens plus those the select kernel recomputed itself.
__global__ void report_uncertified_kernel(const int32_t* __restrict__ nlist,
                                          int32_t* __restrict__ uncertified) {
  *uncertified = nlist[0] + nlist[1];
}
constexpr int kSelThreads = kSelWaves * kWave;
constexpr int kFbThreads = 1024;  // threads per uncertified token in the fallback

// One wave per token. With NOISE, `part` holds 2E columns per token (the router's, then the
// noise rows') and `noise` the (T, E) draw. Without `renorm` every token is listed for the
// exact path (its gates need all E logits exactly); the loss probabilities still come from
// the folded logits here.
template <int EPL, int CG, bool NOISE>
__global__ __launch_bounds__(kSelThreads) void route_select_kernel(
    int64_t T, int64_t D, int E, int k, int S, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ wt, const double* __restrict__ wnorm,
    const float* __restrict__ part, const float* __restrict__ xsq, const float* __restrict__ bias,
    const float* __restrict__ noise, bool renorm, int32_t* __restrict__ idx,
    float* __restrict__ gates, float* __restrict__ logits_out, double* __restrict__ psum_blk,
    int32_t* __restrict__ count_blk, int32_t* __restrict__ list, int32_t* __restrict__ nlist) {
  const int lane = lane_id(), wv = wave_id();
  const int64_t t = (int64_t)blockIdx.x * kRouteTokensPerBlock + wv;
  const bool valid = t < T;
  const int ldp = NOISE ? 2 * E : E;
  double wmax = 0.0, wmaxn = 0.0;  // max_e |W_e| and max_e |W_noise_e|: a wave max each
  for (int e = lane; e < E; e += kWave) {
    wmax = fmax(wmax, wnorm[e]);
    if (NOISE) wmaxn = fmax(wmaxn, wnorm[E + e]);
  }
  wmax = wave_max(wmax);
  if (NOISE) wmaxn = wave_max(wmaxn);

  double lg[EPL], prob[EPL], my_v[EPL];
  int my_e[EPL];
  bool sel[EPL];
  bool flagged = false;
#pragma unroll
  for (int i = 0; i < EPL; ++i) lg[i] = 0.0;
  if (valid) {
    double rnd = 0.0, rndz = 0.0, xn2 = 0.0, ab[EPL], z[EPL], abz[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      ab[i] = 0.0;
      z[i] = 0.0;
      abz[i] = 0.0;
    }
    // partials in split order; 4 splits' loads issued together
    for (int s0 = 0; s0 < S; s0 += 4) {
      float pv[4][EPL], pz[4][EPL], xv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = s0 + q < S;
        xv[q] = ok ? xsq[(int64_t)(s0 + q) * T + t] : 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          const int e = lane + kWave * i;
          const float* row = part + ((int64_t)(s0 + q) * T + t) * ldp;
          pv[q][i] = (ok && e < E) ? row[e] : 0.f;
          pz[q][i] = (NOISE && ok && e < E) ? row[E + e] : 0.f;
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xn2 += (double)xv[q];
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          lg[i] += (double)pv[q][i];
          ab[i] += fabs((double)pv[q][i]);
          if (NOISE) {
            z[i] += (double)pz[q][i];
            abz[i] += fabs((double)pz[q][i]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      rnd = fmax(rnd, ab[i]);
      if (NOISE) rndz = fmax(rndz, abz[i]);
    }
    add_bias<EPL>(bias, E, lg);
    rnd = wave_max(rnd);
    // |computed - exact| bound: every 32-term MFMA sum within 32 * 2^-23 of its sum of
    // |products|, summed by Cauchy-Schwarz; the float32 sum of squares padded by D * 2^-23;
    // the float32 rounding of each partial; the float64 additions.
    const double gamma = 32.0 * 0x1p-23;
    const double xnb = sqrt(xn2 * (1.0 + (double)D * 0x1p-23)) * (1.0 + 1e-6);
    double bnoise = 0.0;
    if (NOISE) {
      rndz = wave_max(rndz);
      double zmax = 0.0;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i < E) zmax = fmax(zmax, fabs(z[i]));
      zmax = wave_max(zmax);
      const double Bz = gamma * xnb * wmaxn + rndz * 0x1p-23 + zmax * 0x1p-50 + 1e-30;
      // noise[t, e] * softplus(z): softplus is 1-Lipschitz, so its error is at most Bz plus
      // its own float64 evaluation; then the product and the sum round once each
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        if (e < E) {
          const double n = (double)noise[t * E + e];
          const double sp = softplus_f64(z[i]);
          lg[i] += n * sp;
          bnoise = fmax(bnoise, fabs(n) * (Bz + (sp + 1.0) * 0x1p-50) +
                                    fabs(n * sp) * 0x1p-52 + fabs(lg[i]) * 0x1p-52);
        }
      }
      bnoise = wave_max(bnoise);
    }
    double lmax = 0.0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i < E) lmax = fmax(lmax, fabs(lg[i]));
    lmax = wave_max(lmax);
    const double B = gamma * xnb * wmax + rnd * 0x1p-23 + lmax * 0x1p-50 + 1e-30 + bnoise;
    const double gap = topk_rounds_keys<EPL>(E, k, lg, sel, my_v, my_e);
    flagged = !renorm || !(gap > 2.0 * B + lmax * 0x1p-22);
    if (flagged && EPL == 1 && E <= kInWaveExact) {
      // few experts: this wave takes all E logits exactly (exact bf16 products, float64
      // sums; with noise also the E noise rows, + noise * softplus) and decides from them,
      // as the fallback would
      double ex = 0.0, zx = 0.0;
      token_dots_f64<8>(x, wt, t, D, NOISE ? 2 * E : E, [](int j) { return j; },
                        [&](int j, double v) {
                          if (j == lane) ex = v;
                          if (NOISE && j - E == lane) zx = v;
                        });
      lg[0] = ex;
      add_bias<EPL>(bias, E, lg);
      if (NOISE && lane < E) lg[0] += (double)noise[t * E + lane] * softplus_f64(zx);
      topk_rounds<EPL>(E, k, lg, sel, my_v, my_e, false);
      flagged = false;
      if (lane == 0) atomicAdd(nlist + 1, 1);
    } else if (flagged) {
      // decided (or, without renormalisation, finished) by route_fallback_kernel from
      // exact logits
      if (lane == 0) list[atomicAdd(nlist, 1)] = (int32_t)t;
    } else if (NOISE) {
      chosen_logits_noisy_f64<EPL, CG>(x, wt, bias, noise, t, D, E, k, my_e, my_v);
    } else {
      chosen_logits_f64<EPL, CG>(x, wt, bias, t, D, k, my_e, my_v);
    }
  }
  BlockPartials<EPL> bp;
  bp.zero();
  if (valid) {
    write_logits<EPL>(logits_out, t, E, lg);
    // (renorm is false only for tokens recomputed in this wave; listed ones are rewritten
    // by the fallback)
    finish_token<EPL>(E, k, t, lg, my_v, my_e, prob, idx, gates, renorm || flagged);
    // the loss probabilities come from these logits for every token; the counts of a
    // listed token are added by the fallback once its experts are known
    if (flagged)
#pragma unroll
      for (int i = 0; i < EPL; ++i) sel[i] = false;
    bp.add(prob, sel);
  }
  write_block_partials<kSelWaves, EPL>(bp, E, psum_blk, count_blk);
}

// Listed tokens (uncertified, or every token without renormalisation), one per 1024-thread
// block at a time: thread i takes router row i / P (the E experts' rows, then with noise their
// E noise rows) and every P-th 16-byte slice of D from slice i % P (P = 1024 / the row count
// rounded up to a power of two), so the exact-product float64 dot products of all rows come
// from 1024 concurrent partial sums, added per row in slice order. Wave 0 then forms the
// logits (plus noise[t, e] * softplus(noise row) with noise), takes the top-k and the gates
// from them and adds the token's counts to its routing block's partials (integer atomics: the
// totals do not depend on order). Also reports the number of listed tokens.
template <int EPL, bool NOISE>
__global__ __launch_bounds__(kFbThreads) void route_fallback_kernel(
    int64_t D, int E, int k, int64_t nblk, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ wt, const float* __restrict__ bias,
    const float* __restrict__ noise, bool renorm, const int32_t* __restrict__ list,
    const int32_t* __restrict__ nlist, int32_t* __restrict__ idx, float* __restrict__ gates,
    float* __restrict__ logits_out, int32_t* __restrict__ count_blk,
    int32_t* __restrict__ uncertified) {
  __shared__ double s_red[kFbThreads];
  __shared__ double s_lg[2 * kMaxExperts];
  const int n = nlist[0];
  if (blockIdx.x == 0 && threadIdx.x == 0 && uncertified) *uncertified = n + nlist[1];
  const int rows = NOISE ? 2 * E : E;
  int NE = 1;
  while (NE < rows) NE <<= 1;
  const int P = kFbThreads / NE;
  const int i = threadIdx.x, pp = i % P, e = i / P;
  const int lane = lane_id();
  for (int slot = blockIdx.x; slot < n; slot += gridDim.x) {
    const int64_t t = list[slot];
    const uint4* xr = (const uint4*)(x + t * D);
    double acc = 0.0;
    if (e < rows) {
      const uint4* wr = (const uint4*)(wt + (int64_t)e * D);
#pragma unroll 4
      for (int64_t c = pp; c < D / 8; c += P) acc += dot8_f64(xr[c], wr[c]);
    }
    s_red[i] = acc;
    __syncthreads();
    if (i < rows) {
      double v = 0.0;
      for (int q = 0; q < P; ++q) v += s_red[i * P + q];
      s_lg[i] = v;
    }
    __syncthreads();
    if (wave_id() == 0) {
      double lg[EPL], prob[EPL], my_v[EPL];
      int my_e[EPL];
      bool sel[EPL];
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        const int ee = lane + kWave * q;
        lg[q] = (ee < E) ? s_lg[ee] : 0.0;
      }
      add_bias<EPL>(bias, E, lg);
      if (NOISE) {
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
          const int ee = lane + kWave * q;
          if (ee < E) lg[q] += (double)noise[t * E + ee] * softplus_f64(s_lg[E + ee]);
        }
      }
      write_logits<EPL>(logits_out, t, E, lg);
      topk_rounds<EPL>(E, k, lg, sel, my_v, my_e, false);
      finish_token<EPL>(E, k, t, lg, my_v, my_e, prob, idx, gates, renorm);
      const int64_t blk = t / kRouteTokensPerBlock;
#pragma unroll
      for (int q = 0; q < EPL; ++q)
        if (sel[q]) atomicAdd(&count_blk[(int64_t)(lane + kWave * q) * nblk + blk], 1);
    }
    __syncthreads();  // s_red / s_lg are reused by the next token
  }
}

// Importance partials: block b (one wave) adds the final gates of its kRouteTokensPerBlock
// tokens per expert, token by token and choice by choice, and writes them expert-major like
// the probability partials.
template <int EPL>
__global__ __launch_bounds__(kWave) void importance_partials_kernel(
    int64_t T, int E, int k, const int32_t* __restrict__ idx, const float* __restrict__ gates,
    double* __restrict__ imp_blk) {
  const int lane = lane_id();
  double acc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc[i] = 0.0;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteTokensPerBlock;
  const int64_t t1 = min(T, t0 + kRouteTokensPerBlock);
  for (int64_t s = t0 * k; s < t1 * k; ++s) {
    const int e = idx[s];
    const double g = (double)gates[s];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (e == lane + kWave * i) acc[i] += g;
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    if (e < E) imp_blk[(int64_t)e * gridDim.x + blockIdx.x] = acc[i];
  }
}

constexpr int kAuxThreads = 256;
static_assert(kAuxThreads >= kMaxExperts, "one thread per expert in the final sum");

// Switch loss from the per-block partials (expert-major, nblk per expert): block e sums
// expert e's probability partials and counts in a fixed order (strided per thread, then a
// fixed tree), writes P_e and count_e, and takes a ticket; the block with the last ticket
// forms aux = E * sum_e (count_e / (T k)) * (P_e / T) (the E terms added by a fixed tree) and
// resets the ticket. With importance partials (imp_blk non-null) each block also sums expert
// e's gate partials, and the last block forms the importance loss, the squared coefficient of
// variation of those E sums (population variance over the squared mean, both fixed trees;
// 0 when nothing was routed).
// The result does not depend on block scheduling.
__global__ __launch_bounds__(kAuxThreads) void aux_finalize_kernel(
    int64_t nblk, int E, int64_t T, int k, const double* __restrict__ psum_blk,
    const int32_t* __restrict__ count_blk, double* __restrict__ pe, int64_t* __restrict__ ce,
    int32_t* __restrict__ ticket, float* __restrict__ aux, int32_t* __restrict__ counts_out,
    const double* __restrict__ imp_blk, double* __restrict__ ie, float* __restrict__ importance) {
  __shared__ double s_p[kAuxThreads];
  __shared__ double s_g[kAuxThreads];
  __shared__ int64_t s_c[kAuxThreads];
  __shared__ bool s_last;
  const int e = blockIdx.x, i = threadIdx.x;
  double pacc = 0.0, gacc = 0.0;
  int64_t cacc = 0;
  const double* pp = psum_blk + (int64_t)e * nblk;
  const int32_t* cp = count_blk + (int64_t)e * nblk;
  const double* gp = imp_blk ? imp_blk + (int64_t)e * nblk : nullptr;
#pragma unroll 4
  for (int64_t b = i; b < nblk; b += kAuxThreads) {
    pacc += pp[b];
    cacc += cp[b];
    if (gp) gacc += gp[b];
  }
  s_p[i] = pacc;
  s_c[i] = cacc;
  s_g[i] = gacc;
  __syncthreads();
  for (int h = kAuxThreads / 2; h >= 1; h >>= 1) {
    if (i < h) {
      s_p[i] += s_p[i + h];
      s_c[i] += s_c[i + h];
      s_g[i] += s_g[i + h];
    }
    __syncthreads();
  }
  if (i == 0) {
    pe[e] = s_p[0];
    ce[e] = s_c[0];
    if (imp_blk) ie[e] = s_g[0];
    if (counts_out) counts_out[e] = (int32_t)s_c[0];
    __threadfence();
    s_last = atomicAdd(ticket, 1) == E - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // thread q forms expert q's term; a fixed tree adds them
  double term = 0.0;
  if (i < E && T > 0) {
    const double Pe = __builtin_nontemporal_load(&pe[i]);
    const double c = (double)__builtin_nontemporal_load(&ce[i]);
    term = (c / ((double)T * (double)k)) * (Pe / (double)T);
  }
  s_p[i] = term;
  __syncthreads();
  for (int h = kAuxThreads / 2; h >= 1; h >>= 1) {
    if (i < h) s_p[i] += s_p[i + h];
    __syncthreads();
  }
  if (i == 0) *aux = (float)((double)E * s_p[0]);
  if (imp_blk) {
    // importance: the mean of the E sums, then the mean squared deviation from it
    const double g = i < E ? __builtin_nontemporal_load(&ie[i]) : 0.0;
    __syncthreads();
    s_g[i] = g;
    __syncthreads();
    for (int h = kAuxThreads / 2; h >= 1; h >>= 1) {
      if (i < h) s_g[i] += s_g[i + h];
      __syncthreads();
    }
    const double mean = s_g[0] / (double)E;
    __syncthreads();
    s_g[i] = i < E ? (g - mean) * (g - mean) : 0.0;
    __syncthreads();
    for (int h = kAuxThreads / 2; h >= 1; h >>= 1) {
      if (i < h) s_g[i] += s_g[i + h];
      __syncthreads();
    }
    if (i == 0) *importance = mean > 0.0 ? (float)((s_g[0] / (double)E) / (mean * mean)) : 0.f;
  }
  if (i == 0) *ticket = 0;
}

__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

// T = 0: aux = 0 (and the importance loss, if asked), every count 0.
__global__ void aux_empty_kernel(int E, float* __restrict__ aux, int32_t* __restrict__ counts_out,
                                 float* __restrict__ importance) {
  if (threadIdx.x == 0) *aux = 0.f;
  if (threadIdx.x == 0 && importance) *importance = 0.f;
  if (counts_out && (int)threadIdx.x < E) counts_out[threadIdx.x] = 0;
}

// ---- scratch layout -------------------------------------------------------------------------

size_t a256(size_t v) { return (v + 255) & ~size_t(255); }

struct RouteScratch {
  double* psum;
  int32_t* pcnt;
  double* pe;        // per-expert probability sums (aux reduction)
  int64_t* ce;       // per-expert counts (aux reduction)
  int32_t* ticket;   // blocks of the aux reduction done; zeroed by the first routing kernel
  int32_t* list;     // uncertified tokens (bf16), appended by the select kernel
  int32_t* nlist;    // [0] their number, [1] the tokens the select kernel recomputed itself;
                     // zeroed by the first routing kernel
  double* imp;       // importance partials (nblk per expert) and ...
  double* ie;        // ... per-expert gate sums
  uint16_t* wt;      // (2E, D): the router's rows, then the noise rows (when there is noise)
  double* wnorm;     // (2E)
  float* part;       // (S, T, 2E) partial logits, router columns then noise columns
  float* xsq;
  size_t bytes;
};

RouteScratch route_scratch(const Problem& p, void* base) {
  RouteScratch r{};
  char* b = (char*)base;
  size_t off = 0;
  auto take = [&](size_t n) {
    char* q = b ? b + off : nullptr;
    off = a256(off + n);
    return q;
  };
  const int64_t nblk = route_blocks(p);
  r.psum = (double*)take((size_t)nblk * p.E * sizeof(double));
  r.pcnt = (int32_t*)take((size_t)nblk * p.E * sizeof(int32_t));
  r.pe = (double*)take((size_t)p.E * sizeof(double));
  r.ce = (int64_t*)take((size_t)p.E * sizeof(int64_t));
  r.ticket = (int32_t*)take(sizeof(int32_t));
  r.list = (int32_t*)take((size_t)p.T * sizeof(int32_t));
  r.nlist = (int32_t*)take(2 * sizeof(int32_t));
  r.imp = (double*)take((size_t)nblk * p.E * sizeof(double));
  r.ie = (double*)take((size_t)p.E * sizeof(double));
  if (p.dtype == MOE_BF16) {  // sized for router noise (2E rows) either way
    const int S = route_splits(p);
    r.wt = (uint16_t*)take((size_t)2 * p.E * p.D * sizeof(uint16_t));
    r.wnorm = (double*)take((size_t)2 * p.E * sizeof(double));
    r.part = (float*)take((size_t)S * p.T * 2 * p.E * sizeof(float));
    r.xsq = (float*)take((size_t)S * p.T * sizeof(float));
  }
  r.bytes = off;
  return r;
}

}  // namespace

int64_t route_blocks(const Problem& p) {
  return (p.T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock;
}

// Splits of the router's K range: enough blocks to fill the chip, each split at least
// kMinKSplit deep, and the float32 partials (written and read back) at most a quarter of
// the bytes of x.
int route_splits(const Problem& p) {
  const int64_t nblk = (p.T + kLT - 1) / kLT;
  int S = 1;
  while (nblk * (2 * S) <= 1024 && p.D / (2 * S) >= kMinKSplit &&
         16 * (int64_t)(2 * S) * p.E <= p.D)
    S *= 2;
  return S;
}

// The fused path's region follows the multi-kernel path's scratch.
size_t route_ws_bytes(const Problem& p) {
  return a256(route_scratch(p, nullptr).bytes) + fused_route_ws_bytes(p);
}
static void* fused_region(const Problem& p, void* ws) {
  return (char*)ws + a256(route_scratch(p, nullptr).bytes);
}

hipError_t launch_route(const Problem& p, const void* x, const void* w_router, const float* bias,
                        const RouteOpts& o, int32_t* idx, float* gates, float* logits_out,
                        int32_t* uncertified, void* ws, hipStream_t s) {
  const RouteScratch r = route_scratch(p, ws);
  const int64_t nblk = route_blocks(p);
  if (nblk == 0) {
    if (uncertified) hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, s, uncertified);
    return hipGetLastError();
  }
  const int epl = (p.E + kWave - 1) / kWave;
  const bool noisy = o.w_noise != nullptr;
  if (p.dtype != MOE_BF16) {
#define MOE_ROUTE_F64(EPLV)                                                                      \
  hipLaunchKernelGGL((route_f64_kernel<float, EPLV>), dim3((unsigned)nblk), dim3(kRouteThreads), \
                     0, s, p.T, p.D, p.E, p.top_k, (const float*)x, (const float*)w_router, bias, \
                     (const float*)o.w_noise, o.noise, o.renorm, idx, gates, logits_out, r.psum, \
                     r.pcnt, r.ticket, uncertified)
    if (epl <= 1)
      MOE_ROUTE_F64(1);
    else if (epl <= 2)
      MOE_ROUTE_F64(2);
    else
      MOE_ROUTE_F64(4);
#undef MOE_ROUTE_F64
    return hipGetLastError();
  }
  const int S = route_splits(p);
  int64_t kc = (p.D + S - 1) / S;
  kc = (kc + 31) / 32 * 32;
  const int rows = noisy ? 2 * p.E : p.E;  // router rows, then noise rows
  hipLaunchKernelGGL(router_prep_kernel, dim3(rows), dim3(256), 0, s, p.D, p.E,
                     (const uint16_t*)w_router, (const uint16_t*)o.w_noise, r.wt, r.wnorm,
                     r.ticket, r.nlist);
  const dim3 lgrid((unsigned)((p.T + kLT - 1) / kLT), (unsigned)S);
  const uint16_t* xb = (const uint16_t*)x;
  // the router product: all rows in one pass when they fit 16 tiles of 16, else the router
  // rows and the noise rows in two passes (the second without the ||x||^2 partials)
  auto logits = [&](int nrows, const uint16_t* w, float* xsq, int col0) {
    const int NT = (nrows + 15) / 16;
    if (NT <= 1)
      hipLaunchKernelGGL(route_logits_mfma_kernel<1>, lgrid, dim3(256), 0, s, p.T, p.D, nrows,
                         kc, xb, w, r.part, xsq, rows, col0);
    else if (NT <= 2)
      hipLaunchKernelGGL(route_logits_mfma_kernel<2>, lgrid, dim3(256), 0, s, p.T, p.D, nrows,
                         kc, xb, w, r.part, xsq, rows, col0);
    else if (NT <= 4)
      hipLaunchKernelGGL(route_logits_mfma_kernel<4>, lgrid, dim3(256), 0, s, p.T, p.D, nrows,
                         kc, xb, w, r.part, xsq, rows, col0);
    else if (NT <= 8)
      hipLaunchKernelGGL(route_logits_mfma_kernel<8>, lgrid, dim3(256), 0, s, p.T, p.D, nrows,
                         kc, xb, w, r.part, xsq, rows, col0);
    else
      hipLaunchKernelGGL(route_logits_mfma_kernel<16>, lgrid, dim3(256), 0, s, p.T, p.D, nrows,
                         kc, xb, w, r.part, xsq, rows, col0);
  };
  if (rows <= 256) {
    logits(rows, r.wt, r.xsq, 0);
  } else {
    logits(p.E, r.wt, r.xsq, 0);
    logits(p.E, r.wt + (int64_t)p.E * p.D, nullptr, p.E);
  }
#define MOE_ROUTE_SELECT(EPLV, CGV, NZ)                                                          \
  hipLaunchKernelGGL((route_select_kernel<EPLV, CGV, NZ>), dim3((unsigned)nblk), dim3(kSelThreads), \
                     0, s, p.T, p.D, p.E, p.top_k, S, xb, r.wt, r.wnorm, r.part, r.xsq, bias,       \
                     o.noise, o.renorm, idx, gates, logits_out, r.psum, r.pcnt, r.list, r.nlist)
#define MOE_ROUTE_SELECT_CG(EPLV, NZ) \
  if (p.top_k <= 2)                   \
    MOE_ROUTE_SELECT(EPLV, 2, NZ);    \
  else if (p.top_k <= 4)              \
    MOE_ROUTE_SELECT(EPLV, 4, NZ);    \
  else if (p.top_k <= 6)              \
    MOE_ROUTE_SELECT(EPLV, 6, NZ);    \
  else                                \
    MOE_ROUTE_SELECT(EPLV, 8, NZ);
#define MOE_ROUTE_SELECT_EPL(NZ) \
  if (epl <= 1) {                \
    MOE_ROUTE_SELECT_CG(1, NZ)   \
  } else if (epl <= 2) {         \
    MOE_ROUTE_SELECT_CG(2, NZ)   \
  } else {                       \
    MOE_ROUTE_SELECT_CG(4, NZ)   \
  }
  if (noisy) {
    MOE_ROUTE_SELECT_EPL(true)
  } else {
    MOE_ROUTE_SELECT_EPL(false)
  }
#undef MOE_ROUTE_SELECT_EPL
#undef MOE_ROUTE_SELECT_CG
#undef MOE_ROUTE_SELECT
  // With E <= kInWaveExact the select kernel lists no token (it recomputes flagged ones
  // itself), so the fallback is skipped and only the count is reported.
  if (epl <= 1 && p.E <= kInWaveExact) {
    if (uncertified)
      hipLaunchKernelGGL(report_uncertified_kernel, dim3(1), dim3(1), 0, s, r.nlist, uncertified);
    return hipGetLastError();
  }
  // one block per listed token, at most 512 blocks (a grid-stride loop covers the rest)
  const unsigned fgrid = (unsigned)std::min<int64_t>(p.T, 512);
#define MOE_ROUTE_FALLBACK(EPLV, NZ)                                                           \
  hipLaunchKernelGGL((route_fallback_kernel<EPLV, NZ>), dim3(fgrid), dim3(kFbThreads), 0, s, \
                     p.D, p.E, p.top_k, nblk, xb, r.wt, bias, o.noise, o.renorm, r.list,      \
                     r.nlist, idx, gates, logits_out, r.pcnt, uncertified)
#define MOE_ROUTE_FALLBACK_EPL(NZ) \
  if (epl <= 1)                    \
    MOE_ROUTE_FALLBACK(1, NZ);     \
  else if (epl <= 2)               \
    MOE_ROUTE_FALLBACK(2, NZ);     \
  else                             \
    MOE_ROUTE_FALLBACK(4, NZ);
  if (noisy) {
    MOE_ROUTE_FALLBACK_EPL(true)
  } else {
    MOE_ROUTE_FALLBACK_EPL(false)
  }
#undef MOE_ROUTE_FALLBACK_EPL
#undef MOE_ROUTE_FALLBACK
  return hipGetLastError();
}

hipError_t launch_aux_finalize(const Problem& p, void* ws, float* aux, int32_t* counts_out,
                               hipStream_t s, const int32_t* idx, const float* gates,
                               float* importance) {
  const RouteScratch r = route_scratch(p, ws);
  const int64_t nblk = route_blocks(p);
  if (nblk == 0) {  // nothing was routed: aux = 0, counts = 0, importance loss 0
    hipLaunchKernelGGL(aux_empty_kernel, dim3(1), dim3(kMaxExperts), 0, s, p.E, aux, counts_out,
                       importance);
    return hipGetLastError();
  }
  if (importance) {
    const int epl = (p.E + kWave - 1) / kWave;
    if (epl <= 1)
      hipLaunchKernelGGL(importance_partials_kernel<1>, dim3((unsigned)nblk), dim3(kWave), 0, s,
                         p.T, p.E, p.top_k, idx, gates, r.imp);
    else if (epl <= 2)
      hipLaunchKernelGGL(importance_partials_kernel<2>, dim3((unsigned)nblk), dim3(kWave), 0, s,
                         p.T, p.E, p.top_k, idx, gates, r.imp);
    else
      hipLaunchKernelGGL(importance_partials_kernel<4>, dim3((unsigned)nblk), dim3(kWave), 0, s,
                         p.T, p.E, p.top_k, idx, gates, r.imp);
  }
  hipLaunchKernelGGL(aux_finalize_kernel, dim3(p.E), dim3(kAuxThreads), 0, s, nblk, p.E, p.T,
                     p.top_k, r.psum, r.pcnt, r.pe, r.ce, r.ticket, aux, counts_out,
                     importance ? r.imp : nullptr, r.ie, importance);
  return hipGetLastError();
}

hipError_t launch_route_full(const Problem& p, const void* x, const void* w_router,
                             const float* bias, const RouteOpts& o, int32_t* idx, float* gates,
                             float* logits_out, int32_t* uncertified, float* aux,
                             int32_t* counts_out, float* importance, void* ws, hipStream_t s,
                             int32_t* offsets_out, bool* dispatch_done) {
  if (dispatch_done) *dispatch_done = false;
  if (fused_route_applies(p, o, importance != nullptr)) {
    hipError_t err =
        launch_route_fused(p, x, w_router, bias, o.renorm, idx, gates, logits_out,
                           fused_region(p, ws), s, importance != nullptr, o.w_noise, o.noise);
    if (err != hipSuccess) return err;
    if (dispatch_done && offsets_out) {
      *dispatch_done = true;  // the caller's launch_place_after_route finishes the loss
      return hipSuccess;
    }
    return launch_place_fused(p, idx, fused_region(p, ws), aux, counts_out, uncertified, nullptr,
                              nullptr, nullptr, s, nullptr, 0, importance);
  }
  hipError_t err = launch_route(p, x, w_router, bias, o, idx, gates, logits_out, uncertified, ws, s);
  if (err == hipSuccess)
    err = launch_aux_finalize(p, ws, aux, counts_out, s, idx, gates, importance);
  return err;
}

hipError_t launch_place_after_route(const Problem& p, const int32_t* idx, void* ws, float* aux,
                                    int32_t* counts_out, int32_t* uncertified,
                                    int32_t* offsets, int32_t* perm, int32_t* slot_row,
                                    hipStream_t s, int32_t* zero, int nzero, float* importance) {
  return launch_place_fused(p, idx, fused_region(p, ws), aux, counts_out, uncertified, offsets,
                            perm, slot_row, s, zero, nzero, importance);
}

}  // namespace moe

// Wave-level pieces of the routing selection, shared by the routing kernels: one wavefront
// per token, lane l holding experts l, l + 64, l + 128, l + 192 (EPL of them, E <= 256).
// Top-k by descending logit with ties to the lower expert index (ML Grind "Mixture-of-Experts
// (MoE) Routing", Algorithm step 2 and "Edge cases and conventions"), the row softmax and the
// gates as the softmax of the chosen logits (Algorithm steps 1 and 2).
#pragma once

#include <float.h>
#include <limits.h>
#include <math.h>

#include "common.hpp"

namespace moe {
namespace {

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xf, 0xf, true);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, true);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  return __longlong_as_double((long long)readlane64((uint64_t)__double_as_longlong(v), l));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  return __longlong_as_double((long long)dpp64<CTRL>((uint64_t)__double_as_longlong(v)));
}

// Wave-wide reductions with the same value, bit for bit, in every lane: within each row of 16
// lanes by four DPP exchanges (lane ^ 1, lane ^ 2, the mirrored lane of the half row, of the
// row; each pairs two lanes that then hold the same result), then the four row results read out
// and combined in a fixed order.
__device__ __forceinline__ double wave_max(double v) {
  v = fmax(v, dpp_f64<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmax(v, dpp_f64<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmax(v, dpp_f64<0x141>(v));  // row_half_mirror
  v = fmax(v, dpp_f64<0x140>(v));  // row_mirror
  const double r0 = readlane_f64(v, 0), r1 = readlane_f64(v, 16);
  const double r2 = readlane_f64(v, 32), r3 = readlane_f64(v, 48);
  return fmax(fmax(r0, r1), fmax(r2, r3));
}
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  const double r0 = readlane_f64(v, 0), r1 = readlane_f64(v, 16);
  const double r2 = readlane_f64(v, 32), r3 = readlane_f64(v, 48);
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ double dot8_f64(const uint4& xv, const uint4& wv) {
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
  const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
  double a = 0.0, b = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    a = fma((double)__uint_as_float(xw[q] << 16), (double)__uint_as_float(ww[q] << 16), a);
    b = fma((double)__uint_as_float(xw[q] & 0xffff0000u),
            (double)__uint_as_float(ww[q] & 0xffff0000u), b);
  }
  return a + b;
}

// k rounds of a wave-wide argmax over the not-yet-chosen experts: larger logit first,
// equal logits -> smaller expert index. Lane j (+64i) keeps the j-th choice. When
// `want_gap`, one more round finds the best unchosen logit, and the smallest difference
// between consecutive values of the chosen sequence (extended by that one) is returned.
template <int EPL>
__device__ __forceinline__ double topk_rounds(int E, int k, const double lg[EPL], bool sel[EPL],
                                              double my_v[EPL], int my_e[EPL],
                                              bool want_gap) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    sel[i] = false;
    my_v[i] = 0.0;
    my_e[i] = 0;
  }
  double prev = 0.0, min_gap = DBL_MAX;
  const int rounds = (want_gap && k < E) ? k + 1 : k;
  for (int j = 0; j < rounds; ++j) {
    double bv = -DBL_MAX;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !sel[i] && (lg[i] > bv || (lg[i] == bv && e < be))) {
        bv = lg[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
      const double ov = __shfl_xor(bv, o);
      const int oe = __shfl_xor(be, o);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if (j > 0) min_gap = fmin(min_gap, prev - bv);
    prev = bv;
    if (j == k) break;  // the extra round only measures the boundary gap
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (be == lane + kWave * i) sel[i] = true;
      if (j == lane + kWave * i) {
        my_v[i] = bv;
        my_e[i] = be;
      }
    }
  }
  return min_gap;
}

// Wave-wide maximum of a 64-bit key, the same in every lane: within each row of 16 lanes by
// four DPP exchanges (lanes l ^ 1, l ^ 2, then the mirrored lane of the half row and of the
// row), then the four row maxima read out.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t m) {
  uint64_t o;
  o = dpp64<0xB1>(m);   // quad_perm [1,0,3,2]
  m = o > m ? o : m;
  o = dpp64<0x4E>(m);   // quad_perm [2,3,0,1]
  m = o > m ? o : m;
  o = dpp64<0x141>(m);  // row_half_mirror
  m = o > m ? o : m;
  o = dpp64<0x140>(m);  // row_mirror
  m = o > m ? o : m;
  const uint64_t r0 = readlane64(m, 0), r1 = readlane64(m, 16);
  const uint64_t r2 = readlane64(m, 32), r3 = readlane64(m, 48);
  const uint64_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// The same selection as topk_rounds with want_gap, for the certified fast path: each round's
// argmax runs on 64-bit keys (the logit rounded to float32, mapped to an order-preserving
// unsigned integer, above the complemented expert index, so equal keys go to the lower index),
// and the chosen expert's float64 value is read from its lane. Rounding to float32 can only
// reorder logits that lie within one float32 ulp of each other; the gaps returned are float64
// differences of the chosen sequence, and the caller's certification threshold includes two
// float32 ulps of the largest logit, so any such token is sent to the exact path.
template <int EPL>
__device__ __forceinline__ double topk_rounds_keys(int E, int k, const double lg[EPL],
                                                   bool sel[EPL], double my_v[EPL],
                                                   int my_e[EPL]) {
  const int lane = lane_id();
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    const uint32_t u = __float_as_uint((float)lg[i]);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    key[i] = e < E ? (((uint64_t)o << 32) | (0xFFFFFFFFu - (uint32_t)e)) : 0ull;
    sel[i] = false;
    my_v[i] = 0.0;
    my_e[i] = 0;
  }
  double prev = 0.0, min_gap = DBL_MAX;
  const int rounds = k < E ? k + 1 : k;
  for (int j = 0; j < rounds; ++j) {
    uint64_t best = 0;
    double cand = 0.0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (!sel[i] && key[i] > best) {
        best = key[i];
        cand = lg[i];
      }
    const uint64_t w = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)w);
    const double bv = readlane_f64(cand, e & (kWave - 1));
    if (j > 0) min_gap = fmin(min_gap, prev - bv);
    prev = bv;
    if (j == k) break;  // the extra round only measures the boundary gap
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (e == lane + kWave * i) sel[i] = true;
      if (j == lane + kWave * i) {
        my_v[i] = bv;
        my_e[i] = e;
      }
    }
  }
  return min_gap;
}

// Probabilities over all experts (returned in prob[]), and the index/gate rows: the gates are
// the softmax of the chosen logits my_v when `renorm`, else the chosen experts' probabilities.
template <int EPL>
__device__ __forceinline__ void finish_token(int E, int k, int64_t t, const double lg[EPL],
                                             const double my_v[EPL], const int my_e[EPL],
                                             double prob[EPL], int32_t* __restrict__ idx,
                                             float* __restrict__ gates, bool renorm = true) {
  const int lane = lane_id();
  double m = -DBL_MAX;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + kWave * i < E) m = fmax(m, lg[i]);
  m = wave_max(m);
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    prob[i] = (lane + kWave * i < E) ? exp(lg[i] - m) : 0.0;
    s += prob[i];
  }
  s = wave_sum(s);
#pragma unroll
  for (int i = 0; i < EPL; ++i) prob[i] /= s;
  if (!renorm) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int j = lane + kWave * i;
      // the probability of choice j's expert, read from the lane that holds that expert
      double pv = 0.0;
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        const double c = __shfl(prob[q], my_e[i] & (kWave - 1));
        if ((my_e[i] >> 6) == q) pv = c;
      }
      if (j < k) {
        idx[t * k + j] = my_e[i];
        gates[t * k + j] = (float)pv;
      }
    }
    return;
  }
  // gates: softmax over the chosen logits, shifted by the first (largest) of them
  const double v0 = readlane_f64(my_v[0], 0);
  double ev[EPL];
  double gs = 0.0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    ev[i] = (lane + kWave * i < k) ? exp(my_v[i] - v0) : 0.0;
    gs += ev[i];
  }
  gs = wave_sum(gs);
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int j = lane + kWave * i;
    if (j < k) {
      idx[t * k + j] = my_e[i];
      gates[t * k + j] = (float)(ev[i] / gs);
    }
  }
}

template <int EPL>
__device__ __forceinline__ void add_bias(const float* __restrict__ bias, int E, double lg[EPL]) {
  if (!bias) return;
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    if (e < E) lg[i] += (double)bias[e];
  }
}

template <int EPL>
__device__ __forceinline__ void write_logits(float* __restrict__ logits_out, int64_t t, int E,
                                             const double lg[EPL]) {
  if (!logits_out) return;
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    if (e < E) logits_out[t * E + e] = (float)lg[i];
  }
}

}  // namespace
}  // namespace moe

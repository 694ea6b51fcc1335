// Routing: router logits, row softmax, top-k by descending logit, gates = softmax of the
// k chosen logits, and the per-block partial sums the Switch loss needs.
// (ML Grind "Mixture-of-Experts (MoE) Routing", Algorithm steps 1 and 2 and the
// load-balancing step; ties go to the lower expert index, "Edge cases and conventions".)
//
// One wavefront owns one token at a time; lane l holds experts l, l+64, l+128, l+192
// (E <= 256), so the softmax and the top-k are wave-wide shuffles over registers.
// Logits here are accumulated in float64 from exactly widened inputs: the products of two
// float32 (or bfloat16) values are exact in float64, so these logits are within a few
// float64 ulps of the exact ones.
#include <float.h>
#include <limits.h>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kEPL = kMaxExperts / kWave;  // experts per lane
constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

// xor-butterfly sum: every lane ends with the same, order-fixed value.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename TIn>
__device__ __forceinline__ void logits_f64(const TIn* __restrict__ x, const TIn* __restrict__ w,
                                           const float* __restrict__ bias, int64_t t, int64_t D,
                                           int E, double lg[kEPL]) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < kEPL; ++i) lg[i] = 0.0;
  const TIn* xr = x + t * D;
  for (int64_t d = 0; d < D; ++d) {
    const double xv = load_as_f64(xr, d);
    const TIn* wr = w + d * E;
#pragma unroll
    for (int i = 0; i < kEPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E) lg[i] = fma(xv, load_as_f64(wr, e), lg[i]);
    }
  }
  if (bias) {
#pragma unroll
    for (int i = 0; i < kEPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E) lg[i] += (double)bias[e];
    }
  }
}

// Softmax over all E logits (probabilities, for the loss) and the top-k selection with
// gates. Writes the token's index and gate rows; returns its probabilities and the
// selection mask in registers.
__device__ __forceinline__ void select_token(int E, int k, int64_t t, const double lg[kEPL],
                                             double prob[kEPL], bool sel[kEPL],
                                             int32_t* __restrict__ idx,
                                             float* __restrict__ gates) {
  const int lane = lane_id();
  double m = -DBL_MAX;
#pragma unroll
  for (int i = 0; i < kEPL; ++i)
    if (lane + kWave * i < E) m = fmax(m, lg[i]);
  m = wave_max(m);
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kEPL; ++i) {
    prob[i] = (lane + kWave * i < E) ? exp(lg[i] - m) : 0.0;
    s += prob[i];
    sel[i] = false;
  }
  s = wave_sum(s);
#pragma unroll
  for (int i = 0; i < kEPL; ++i) prob[i] /= s;

  // k rounds of a wave-wide argmax over the not-yet-chosen experts:
  // larger logit first, equal logits -> smaller expert index.
  double my_v[kEPL];
  int my_e[kEPL];
#pragma unroll
  for (int i = 0; i < kEPL; ++i) {
    my_v[i] = 0.0;
    my_e[i] = 0;
  }
  double v0 = 0.0;
  for (int j = 0; j < k; ++j) {
    double bv = -DBL_MAX;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < kEPL; ++i) {
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
    if (j == 0) v0 = bv;
#pragma unroll
    for (int i = 0; i < kEPL; ++i) {
      if (be == lane + kWave * i) sel[i] = true;
      if (j == lane + kWave * i) {
        my_v[i] = bv;
        my_e[i] = be;
      }
    }
  }
  // gates: softmax over the chosen logits (max = the first chosen one)
  double ev[kEPL];
  double gs = 0.0;
#pragma unroll
  for (int i = 0; i < kEPL; ++i) {
    ev[i] = (lane + kWave * i < k) ? exp(my_v[i] - v0) : 0.0;
    gs += ev[i];
  }
  gs = wave_sum(gs);
#pragma unroll
  for (int i = 0; i < kEPL; ++i) {
    const int j = lane + kWave * i;
    if (j < k) {
      idx[t * k + j] = my_e[i];
      gates[t * k + j] = (float)(ev[i] / gs);
    }
  }
}

template <typename TIn>
__global__ __launch_bounds__(kRouteThreads) void route_f64_kernel(
    int64_t T, int64_t D, int E, int k, const TIn* __restrict__ x, const TIn* __restrict__ w,
    const float* __restrict__ bias, int32_t* __restrict__ idx, float* __restrict__ gates,
    float* __restrict__ logits_out, double* __restrict__ psum_blk,
    int32_t* __restrict__ count_blk) {
  __shared__ double s_psum[kRouteWaves][kMaxExperts];
  __shared__ int s_cnt[kRouteWaves][kMaxExperts];
  const int wv = wave_id(), lane = lane_id();
  double psum[kEPL];
  int cnt[kEPL];
#pragma unroll
  for (int i = 0; i < kEPL; ++i) {
    psum[i] = 0.0;
    cnt[i] = 0;
  }
  const int64_t t0 = (int64_t)blockIdx.x * kRouteTokensPerBlock;
  for (int q = wv; q < kRouteTokensPerBlock; q += kRouteWaves) {
    const int64_t t = t0 + q;
    if (t >= T) break;
    double lg[kEPL], prob[kEPL];
    bool sel[kEPL];
    logits_f64(x, w, bias, t, D, E, lg);
    if (logits_out) {
#pragma unroll
      for (int i = 0; i < kEPL; ++i) {
        const int e = lane + kWave * i;
        if (e < E) logits_out[t * E + e] = (float)lg[i];
      }
    }
    select_token(E, k, t, lg, prob, sel, idx, gates);
#pragma unroll
    for (int i = 0; i < kEPL; ++i) {
      psum[i] += prob[i];
      cnt[i] += sel[i] ? 1 : 0;
    }
  }
#pragma unroll
  for (int i = 0; i < kEPL; ++i) {
    s_psum[wv][lane + kWave * i] = psum[i];
    s_cnt[wv][lane + kWave * i] = cnt[i];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    double a = 0.0;
    int c = 0;
#pragma unroll
    for (int q = 0; q < kRouteWaves; ++q) {
      a += s_psum[q][e];
      c += s_cnt[q][e];
    }
    psum_blk[(int64_t)blockIdx.x * E + e] = a;
    count_blk[(int64_t)blockIdx.x * E + e] = c;
  }
}

// aux = E * sum_e (count_e / (T k)) * (sum_t probs[t, e] / T), partials summed in block order.
__global__ __launch_bounds__(kMaxExperts) void aux_finalize_kernel(
    int64_t nblk, int E, int64_t T, int k, const double* __restrict__ psum_blk,
    const int32_t* __restrict__ count_blk, float* __restrict__ aux,
    int32_t* __restrict__ counts_out) {
  __shared__ double s_term[kMaxExperts];
  const int e = threadIdx.x;
  if (e < E) {
    double P = 0.0;
    int64_t c = 0;
    for (int64_t b = 0; b < nblk; ++b) {
      P += psum_blk[b * E + e];
      c += count_blk[b * E + e];
    }
    if (counts_out) counts_out[e] = (int32_t)c;
    s_term[e] = (T > 0) ? ((double)c / ((double)T * (double)k)) * (P / (double)T) : 0.0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int q = 0; q < E; ++q) s += s_term[q];
    *aux = (float)((double)E * s);
  }
}

}  // namespace

int64_t route_blocks(const Problem& p) {
  return (p.T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock;
}

hipError_t launch_route(const Problem& p, const void* x, const void* w_router, const float* bias,
                        int32_t* idx, float* gates, float* logits_out, double* psum_blk,
                        int32_t* count_blk, hipStream_t s) {
  const int64_t nblk = route_blocks(p);
  if (nblk == 0) return hipSuccess;
  if (p.dtype == MOE_BF16) {
    hipLaunchKernelGGL(route_f64_kernel<uint16_t>, dim3((unsigned)nblk), dim3(kRouteThreads), 0,
                       s, p.T, p.D, p.E, p.top_k, (const uint16_t*)x, (const uint16_t*)w_router,
                       bias, idx, gates, logits_out, psum_blk, count_blk);
  } else {
    hipLaunchKernelGGL(route_f64_kernel<float>, dim3((unsigned)nblk), dim3(kRouteThreads), 0, s,
                       p.T, p.D, p.E, p.top_k, (const float*)x, (const float*)w_router, bias, idx,
                       gates, logits_out, psum_blk, count_blk);
  }
  return hipGetLastError();
}

hipError_t launch_aux_finalize(const Problem& p, const double* psum_blk, const int32_t* count_blk,
                               float* aux, int32_t* counts_out, hipStream_t s) {
  hipLaunchKernelGGL(aux_finalize_kernel, dim3(1), dim3(kMaxExperts), 0, s, route_blocks(p), p.E,
                     p.T, p.top_k, psum_blk, count_blk, aux, counts_out);
  return hipGetLastError();
}

}  // namespace moe

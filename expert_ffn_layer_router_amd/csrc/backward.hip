// Backward of the layer: the gradients of L = sum(out * dout) + d_aux * aux_loss with respect
// to x, the router (weights, bias) and every expert matrix. The routing decisions (top-k, the
// drop set) are piecewise constant, so the gradient flows through the gates and through P in
// the Switch loss; f, a count, is a step function of the logits and has none ("Mixture-of-
// Experts (MoE) Routing", the load-balancing step; "Mixture of Experts: the Sparsely-Gated
// Layer", Hot shards). In reverse order of the forward:
//  * combine:  dgate[t, j] = <dout[t], y[row]> for a kept slot (0 for a dropped one),
//              dy[row] = gate[t, j] * dout[t]. For bf16 ReLU / SwiGLU layers the same
//              dgate is taken as <dout[t] W2^T, h[row]> in the activation backward, so y
//              is never needed;
//  * experts:  dh = dy W2^T, then through the activation (ReLU: relu'(0) = 0; SwiGLU:
//              silu'(a) = s (1 + a (1 - s)), s = sigmoid(a)); dx_rows = da W1^T (+ db W3^T);
//              dW2 = h^T dy, dW1 = x^T da (, dW3 = x^T db), each over the expert's kept rows;
//  * gates:    softmax over the k chosen logits: dl_c = g_c (dg_c - sum_c' g_c' dg_c');
//  * loss:     aux = E sum_e f_e P_e, P_e = mean_t p[t, e]: dL/dp[t, e] = d_aux E f_e / T, then
//              through the full softmax: dl[t, e] += p[t, e] (a_e - sum_j p[t, j] a_j);
//  * router:   dW_router = x^T dl, dbias = sum_t dl, dx += dl W_router^T.
// The forward quantities it needs (decisions, gates, logits, the experts' pre-activations,
// h, and y where it is used) are recomputed with the forward's own kernels, so the call needs
// only the inputs and dout; or they come from a training forward's saved state. Every
// reduction runs in a fixed order, so the result does not depend on scheduling.
//
// GEMM shapes that the forward does not have get their own kernels (bf16: 128 x 128 tiles,
// 2 x 2 waves of 64 x 64, v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//  * NT, dgrad: C[r, n] = sum_k A[r, k] W_e[n, k] over each expert's rows r (the tile
//    schedule from the offsets, as in the forward); the weights are read as (E, N, K), i.e.
//    the forward's (in, out) matrices used transposed. Two (A, W) pairs can share one K loop
//    (da W1^T + db W3^T).
//  * TN, wgrad: C_e[m, n] = sum over expert e's rows r of A[r, m] B[r, n]; K is the expert's
//    row count. Both operands are row-major with m / n contiguous, so both are transposed on
//    their way into LDS (4 rows x 8 columns per thread, repacked in registers). A's rows can
//    be gathered (token rows of x through the permutation).
#include <algorithm>

#include "common.hpp"
#include "tile_schedule.hpp"

namespace moe {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLds = kBK + 8;  // padded row stride (elements) of the LDS tiles
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xffffu; }

// 8 bf16 (one 16-byte vector) to float32 and back (round to nearest even).
__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }

struct BwdGemm {
  const void* A0;        // NT: (rows, K) row-major; TN: (rows, M) row-major (gathered)
  const void* A1;        // NT: second A (same shape), or null
  const void* W0;        // NT: (E, N, K) row-major
  const void* W1;        // NT: second W, or null
  const void* B;         // TN: (rows, N) row-major
  const int32_t* gather; // TN: A row of r is gather[r] / gather_div (null: r)
  int gather_div;
  const int32_t* offsets;
  int E;
  int64_t K, M, N;       // NT: K and N (M = rows); TN: M and N (K = rows of the expert)
  int64_t lda;           // row stride of A (elements)
  void* C;               // NT: (rows, N); TN: (E, M, N)
  int64_t max_rows;
};

template <typename OutT>
__device__ __forceinline__ void store_out(OutT* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, int64_t i, float v) {
  p[i] = f32_to_bf16(v);
}

// 4 x 8 block (4 rows of 8 contiguous columns) -> LDS as 8 columns of 4 consecutive rows:
// the transposed layout the MFMA operand wants (K values contiguous per column).
__device__ __forceinline__ void store_transposed(const uint4 (&r)[4], uint16_t* s, int col8,
                                                 int krow4) {
  const uint32_t w0[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
  const uint32_t w1[4] = {r[1].x, r[1].y, r[1].z, r[1].w};
  const uint32_t w2[4] = {r[2].x, r[2].y, r[2].z, r[2].w};
  const uint32_t w3[4] = {r[3].x, r[3].y, r[3].z, r[3].w};
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    const uint32_t lo01 = lo16(w0[wi]) | (lo16(w1[wi]) << 16);
    const uint32_t lo23 = lo16(w2[wi]) | (lo16(w3[wi]) << 16);
    const uint32_t hi01 = hi16(w0[wi]) | (hi16(w1[wi]) << 16);
    const uint32_t hi23 = hi16(w2[wi]) | (hi16(w3[wi]) << 16);
    *(uint2*)&s[(8 * col8 + 2 * wi) * kLds + 4 * krow4] = make_uint2(lo01, lo23);
    *(uint2*)&s[(8 * col8 + 2 * wi + 1) * kLds + 4 * krow4] = make_uint2(hi01, hi23);
  }
}

// One 64-deep slice of MFMAs on the LDS tiles (2 x 2 tiles of 32 x 32 per wave).
__device__ __forceinline__ void mfma_slice(const uint16_t* sA, const uint16_t* sB,
                                           f32x16 (&acc)[2][2], int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < kBK; kk += 16) {
    bf16x8 a[2], b[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
      a[mi] = *(const bf16x8*)&sA[(wm * 64 + mi * 32 + (lane & 31)) * kLds + kk + (lane >> 5) * 8];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
      b[ni] = *(const bf16x8*)&sB[(wn * 64 + ni * 32 + (lane & 31)) * kLds + kk + (lane >> 5) * 8];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
  }
}

// NT (dgrad): grid (M-tiles of all experts, N-tiles). NSEG pairs (A_s, W_s) over the same K.
template <int NSEG, typename OutT>
__global__ __launch_bounds__(kThreads, 2) void nt_bf16_kernel(const BwdGemm g) {
  __shared__ __align__(16) uint16_t sA[kBM * kLds];
  __shared__ __align__(16) uint16_t sB[kBN * kLds];
  int e, row0, rows;
  if (!find_tile(g.offsets, g.E, kBM, (int)blockIdx.x, e, row0, rows)) return;
  const int64_t K = g.K, N = g.N;
  const int64_t n0 = (int64_t)blockIdx.y * kBN;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  const int wm = wv >> 1, wn = wv & 1;
  const int kc = (tid & 7) * 8;  // this thread's 8 K-values within the slice
  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int sg = 0; sg < NSEG; ++sg) {
    const uint16_t* A = (const uint16_t*)(sg ? g.A1 : g.A0);
    const uint16_t* W = (const uint16_t*)(sg ? g.W1 : g.W0) + (int64_t)e * N * K;
    const uint16_t* a_src[4];
    const uint16_t* w_src[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = (tid >> 3) + 32 * p;
      a_src[p] = r < rows ? A + (int64_t)(row0 + r) * g.lda : nullptr;
      w_src[p] = n0 + r < N ? W + (n0 + r) * K : nullptr;
    }
    uint4 ra[4], rb[4];
    auto load = [&](int64_t k0) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const bool ok = k0 + kc < K;  // K % 8 == 0: a vector is all in or all out
        ra[p] = (ok && a_src[p]) ? *(const uint4*)(a_src[p] + k0 + kc) : zero;
        rb[p] = (ok && w_src[p]) ? *(const uint4*)(w_src[p] + k0 + kc) : zero;
      }
    };
    load(0);
    for (int64_t k0 = 0; k0 < K; k0 += kBK) {
      __syncthreads();
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        *(uint4*)&sA[((tid >> 3) + 32 * p) * kLds + kc] = ra[p];
        *(uint4*)&sB[((tid >> 3) + 32 * p) * kLds + kc] = rb[p];
      }
      __syncthreads();
      if (k0 + kBK < K) load(k0 + kBK);
      mfma_slice(sA, sB, acc, wm, wn, lane);
    }
  }
  OutT* C = (OutT*)g.C;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + mi * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        const int64_t col = n0 + wn * 64 + ni * 32 + (lane & 31);
        if (r < rows && col < N) store_out<OutT>(C, (int64_t)(row0 + r) * N + col, acc[mi][ni][v]);
      }
}

// TN (wgrad): grid (M-tiles, N-tiles, experts); K runs over the expert's rows.
template <typename OutT>
__global__ __launch_bounds__(kThreads, 2) void tn_bf16_kernel(const BwdGemm g) {
  __shared__ __align__(16) uint16_t sA[kBM * kLds];
  __shared__ __align__(16) uint16_t sB[kBN * kLds];
  const int e = blockIdx.z;
  const int64_t r0 = g.offsets[e], r1 = g.offsets[e + 1];
  const int64_t M = g.M, N = g.N;
  const int64_t m0 = (int64_t)blockIdx.x * kBM, n0 = (int64_t)blockIdx.y * kBN;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  const int wm = wv >> 1, wn = wv & 1;
  const int kq = tid >> 4, c8 = tid & 15;  // 4 rows from 4 kq, 8 columns from 8 c8
  const int64_t am = m0 + 8 * c8, bn = n0 + 8 * c8;
  const bool a_ok = am < M, b_ok = bn < N;  // M, N % 8 == 0
  const uint16_t* A = (const uint16_t*)g.A0;
  const uint16_t* Bm = (const uint16_t*)g.B;
  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  uint4 ra[4], rb[4];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = r0 + k0 + 4 * kq + i;
      const bool ok = r < r1;
      int64_t src = r;
      if (ok && g.gather) src = g.gather[r] / g.gather_div;
      ra[i] = (ok && a_ok) ? *(const uint4*)(A + src * g.lda + am) : zero;
      rb[i] = (ok && b_ok) ? *(const uint4*)(Bm + r * N + bn) : zero;
    }
  };
  const int64_t K = r1 - r0;
  if (K > 0) load(0);
  for (int64_t k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
    store_transposed(ra, sA, c8, kq);
    store_transposed(rb, sB, c8, kq);
    __syncthreads();
    if (k0 + kBK < K) load(k0 + kBK);
    mfma_slice(sA, sB, acc, wm, wn, lane);
  }
  OutT* C = (OutT*)g.C + (int64_t)e * M * N;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * 64 + mi * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        const int64_t n = n0 + wn * 64 + ni * 32 + (lane & 31);
        if (m < M && n < N) store_out<OutT>(C, m * N + n, acc[mi][ni][v]);
      }
}

// float32 layers: one thread per output element, K in order (the fp32 layers are small).
template <int NSEG>
__global__ __launch_bounds__(kThreads) void nt_f32_kernel(const BwdGemm g) {
  int e, row0, rows;
  if (!find_tile(g.offsets, g.E, 16, (int)blockIdx.x, e, row0, rows)) return;
  const int r = threadIdx.x / 16;
  const int64_t n = (int64_t)blockIdx.y * 16 + (threadIdx.x % 16);
  if (r >= rows || n >= g.N) return;
  float acc = 0.f;
#pragma unroll
  for (int sg = 0; sg < NSEG; ++sg) {
    const float* a = (const float*)(sg ? g.A1 : g.A0) + (int64_t)(row0 + r) * g.lda;
    const float* w = (const float*)(sg ? g.W1 : g.W0) + ((int64_t)e * g.N + n) * g.K;
    for (int64_t k = 0; k < g.K; ++k) acc = fmaf(a[k], w[k], acc);
  }
  ((float*)g.C)[(int64_t)(row0 + r) * g.N + n] = acc;
}

__global__ __launch_bounds__(kThreads) void tn_f32_kernel(const BwdGemm g) {
  const int e = blockIdx.z;
  const int64_t m = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;
  const int64_t n = (int64_t)blockIdx.y * 16 + threadIdx.x % 16;
  if (m >= g.M || n >= g.N) return;
  float acc = 0.f;
  for (int64_t r = g.offsets[e]; r < g.offsets[e + 1]; ++r) {
    const int64_t src = g.gather ? g.gather[r] / g.gather_div : r;
    acc = fmaf(((const float*)g.A0)[src * g.lda + m], ((const float*)g.B)[r * g.N + n], acc);
  }
  ((float*)g.C)[((int64_t)e * g.M + m) * g.N + n] = acc;
}

// ---- elementwise and reduction kernels ------------------------------------------------------

// h = act(a, b) over the kept rows (rows from offsets[E] on are left alone).
// da (and db) from dh, a, b: SwiGLU da = dh b s (1 + a (1 - s)), db = dh a s; ReLU da = dh
// (a > 0).
template <typename TIn>
__global__ void act_backward_kernel(int64_t DH, int kind, const int32_t* __restrict__ offsets,
                                    int E, const TIn* __restrict__ a, const TIn* __restrict__ b,
                                    const TIn* __restrict__ dh, TIn* __restrict__ da,
                                    TIn* __restrict__ db) {
  const int64_t n = (int64_t)offsets[E] * DH;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float av = load_as_f32(a, i), g = load_as_f32(dh, i);
    if (kind == MOE_EXPERT_SWIGLU) {
      const float bv = load_as_f32(b, i);
      const float s = 1.f / (1.f + __expf(-av));
      store_from_f32(da, i, g * bv * s * (1.f + av * (1.f - s)));
      store_from_f32(db, i, g * av * s);
    } else {
      store_from_f32(da, i, av > 0.f ? g : 0.f);
    }
  }
}

// Combine backward, one wave per token: for each of its slots j, dgate = <dout_t, y[row]>
// (float64 sum, lanes over columns then a fixed butterfly) and dy[row] = gate * dout_t, or
// dgate = 0 for a dropped slot.
template <typename TIn>
__global__ __launch_bounds__(kThreads) void combine_backward_kernel(
    int64_t T, int k, int64_t Dout, const TIn* __restrict__ dout, const TIn* __restrict__ y,
    const int32_t* __restrict__ slot_row, const float* __restrict__ gates,
    TIn* __restrict__ dy, float* __restrict__ dgates) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + wave_id();
  if (t >= T) return;
  for (int j = 0; j < k; ++j) {
    const int64_t s = t * k + j;
    const int row = slot_row[s];
    double acc = 0.0;
    if (row >= 0) {
      const float g = gates[s];
      for (int64_t c = lane; c < Dout; c += kWave) {
        const float d = load_as_f32(dout, t * Dout + c);
        acc += (double)d * (double)load_as_f32(y, (int64_t)row * Dout + c);
        store_from_f32(dy, (int64_t)row * Dout + c, g * d);
      }
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) dgates[s] = (float)acc;
  }
}

// The activation backward fused with the gate gradient, one wave per kept row r (slot
// s = perm[r]), for bf16 ReLU / SwiGLU layers with DH % 8 == 0. g = dout_t W2^T (the dgrad of
// the unscaled output gradient); h = act(a, b) from the stored pre-activations; then
// dgate[s] = <g, h> (float64 in column order per lane, then a fixed butterfly), which equals
// <dout_t, h W2> = <dout_t, y>, and with dh = gate * g: SwiGLU da = dh b silu'(a),
// db = dh silu(a); ReLU da = dh [a > 0].
__global__ __launch_bounds__(kThreads) void act_backward_rows_bf16x8_kernel(
    int64_t DH, int kind, const int32_t* __restrict__ offsets, int E,
    const int32_t* __restrict__ perm, const float* __restrict__ gates,
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
    const uint16_t* __restrict__ g, uint16_t* __restrict__ da, uint16_t* __restrict__ db,
    float* __restrict__ dgates) {
  const int64_t r = (int64_t)blockIdx.x * (kThreads / kWave) + wave_id();
  if (r >= offsets[E]) return;
  const int lane = lane_id();
  const int slot = perm[r];
  const float gate = gates[slot];
  const bool swiglu = kind == MOE_EXPERT_SWIGLU;
  double acc = 0.0;
#pragma unroll 2
  for (int64_t c = 8 * lane; c < DH; c += 8 * kWave) {
    const int64_t i = r * DH + c;
    float av[8], gv[8], bv[8], ra[8], rb[8];
    unpack8(*(const uint4*)(a + i), av);
    unpack8(*(const uint4*)(g + i), gv);
    if (swiglu) unpack8(*(const uint4*)(b + i), bv);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float dh = gate * gv[q];
      if (swiglu) {
        const float sg = 1.f / (1.f + __expf(-av[q]));
        const float h = av[q] * sg * bv[q];
        acc += (double)gv[q] * (double)h;
        ra[q] = dh * bv[q] * sg * (1.f + av[q] * (1.f - sg));
        rb[q] = dh * av[q] * sg;
      } else {
        acc += (double)gv[q] * (double)fmaxf(av[q], 0.f);
        ra[q] = av[q] > 0.f ? dh : 0.f;
      }
    }
    *(uint4*)(da + i) = pack8(ra);
    if (swiglu) *(uint4*)(db + i) = pack8(rb);
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) dgates[slot] = (float)acc;
}

// dy[row] = gate[t, j] * dout[t] for each kept slot (bf16, Dout % 8 == 0), and dgate = 0 for
// each dropped slot; one wave per token.
__global__ __launch_bounds__(kThreads) void scale_dout_rows_bf16x8_kernel(
    int64_t T, int k, int64_t Dout, const uint16_t* __restrict__ dout,
    const int32_t* __restrict__ slot_row, const float* __restrict__ gates,
    uint16_t* __restrict__ dy, float* __restrict__ dgates) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + wave_id();
  if (t >= T) return;
  for (int j = 0; j < k; ++j) {
    const int64_t s = t * k + j;
    const int row = slot_row[s];
    if (row < 0) {
      if (lane == 0) dgates[s] = 0.f;
      continue;
    }
    const float gt = gates[s];
    for (int64_t c = 8 * lane; c < Dout; c += 8 * kWave) {
      float d[8], o[8];
      unpack8(*(const uint4*)(dout + t * Dout + c), d);
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = gt * d[q];
      *(uint4*)(dy + (int64_t)row * Dout + c) = pack8(o);
    }
  }
}

// bf16 version of combine_backward, 8 columns a lane (Dout % 8 == 0): lane l takes columns
// 8 (l + 64 i) .. + 7, its float64 partial in column order, then the same butterfly.
__global__ __launch_bounds__(kThreads) void combine_backward_bf16x8_kernel(
    int64_t T, int k, int64_t Dout, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ y, const int32_t* __restrict__ slot_row,
    const float* __restrict__ gates, uint16_t* __restrict__ dy, float* __restrict__ dgates) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + wave_id();
  if (t >= T) return;
  for (int j = 0; j < k; ++j) {
    const int64_t s = t * k + j;
    const int row = slot_row[s];
    double acc = 0.0;
    if (row >= 0) {
      const float g = gates[s];
      for (int64_t c = 8 * lane; c < Dout; c += 8 * kWave) {
        float d[8], yv[8], o[8];
        unpack8(*(const uint4*)(dout + t * Dout + c), d);
        unpack8(*(const uint4*)(y + (int64_t)row * Dout + c), yv);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          acc += (double)d[q] * (double)yv[q];
          o[q] = g * d[q];
        }
        *(uint4*)(dy + (int64_t)row * Dout + c) = pack8(o);
      }
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) dgates[s] = (float)acc;
  }
}

// Router backward, one wave per token (lane l holds experts l + 64 i): probabilities from the
// float32 logits (float64 softmax), then dl over the chosen experts from the gates' softmax and
// over all experts from the loss term.
template <int EPL>
__global__ __launch_bounds__(kThreads) void router_backward_kernel(
    int64_t T, int E, int k, float d_aux, const float* __restrict__ logits,
    const int32_t* __restrict__ idx, const float* __restrict__ gates,
    const float* __restrict__ dgates, const int32_t* __restrict__ counts, float* __restrict__ dl) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + wave_id();
  if (t >= T) return;
  double p[EPL], a[EPL], d[EPL];
  double m = -1e300;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    p[i] = e < E ? (double)logits[t * E + e] : -1e300;
    m = fmax(m, p[i]);
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o));
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    p[i] = e < E ? exp(p[i] - m) : 0.0;
    s += p[i];
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  // loss term: a_e = d_aux * E * f_e / T with f_e = count_e / (T k)
  double pa = 0.0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    p[i] /= s;
    a[i] = e < E ? (double)d_aux * (double)E * ((double)counts[e] / ((double)T * k)) / (double)T
                 : 0.0;
    pa += p[i] * a[i];
    d[i] = 0.0;
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) pa += __shfl_xor(pa, o);
#pragma unroll
  for (int i = 0; i < EPL; ++i) d[i] = p[i] * (a[i] - pa);
  // gates' softmax: dl_c = g_c (dg_c - sum g dg), added at the chosen experts
  double sg = 0.0;
  for (int j = 0; j < k; ++j) sg += (double)gates[t * k + j] * (double)dgates[t * k + j];
  for (int j = 0; j < k; ++j) {
    const int e = idx[t * k + j];
    const double v = (double)gates[t * k + j] * ((double)dgates[t * k + j] - sg);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (e == lane + kWave * i) d[i] += v;
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    if (e < E) dl[t * E + e] = (float)d[i];
  }
}

// dbias[e] = sum_t dl[t, e]: one block per expert, strided partial sums then a fixed tree.
__global__ __launch_bounds__(256) void dbias_kernel(int64_t T, int E, const float* __restrict__ dl,
                                                    float* __restrict__ dbias) {
  __shared__ double s_part[256];
  const int e = blockIdx.x;
  double acc = 0.0;
  for (int64_t t = threadIdx.x; t < T; t += 256) acc += (double)dl[t * E + e];
  s_part[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if ((int)threadIdx.x < h) s_part[threadIdx.x] += s_part[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) dbias[e] = (float)s_part[0];
}

// dW_router[d, e] = sum_t x[t, d] dl[t, e] in two fixed-order levels: block (256 columns d,
// 8 experts, token chunk c of at most kDwrMaxChunk tokens) sums its chunk's tokens in order
// into part[c, d, e], with the chunk's dl rows staged in LDS; then dw_router_reduce adds the
// chunks in order.
constexpr int kDwrMaxChunk = 64;
template <typename TIn>
__global__ __launch_bounds__(256) void dw_router_partial_kernel(int64_t T, int64_t D, int E,
                                                                int64_t tc,
                                                                const TIn* __restrict__ x,
                                                                const float* __restrict__ dl,
                                                                float* __restrict__ part) {
  __shared__ float s_dl[kDwrMaxChunk][8];
  const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = d < D;
  const int e0 = blockIdx.y * 8;
  const int64_t c = blockIdx.z, t0 = c * tc, t1 = min(T, t0 + tc);
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  // the chunk's tokens in order, kDwrMaxChunk dl rows in LDS at a time
  for (int64_t b0 = t0; b0 < t1; b0 += kDwrMaxChunk) {
    __syncthreads();  // the previous rows are no longer read
    for (int i = threadIdx.x; i < kDwrMaxChunk * 8; i += 256) {
      const int64_t t = b0 + i / 8;
      const int e = e0 + i % 8;
      s_dl[i / 8][i % 8] = (t < t1 && e < E) ? dl[t * E + e] : 0.f;
    }
    __syncthreads();
    const int n = (int)min<int64_t>(kDwrMaxChunk, t1 - b0);
    if (valid) {
#pragma unroll 8
      for (int i = 0; i < n; ++i) {
        const float xv = load_as_f32(x, (b0 + i) * D + d);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(xv, s_dl[i][q], acc[q]);
      }
    }
  }
  if (!valid) return;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    if (e0 + q < E) part[(c * D + d) * E + e0 + q] = acc[q];
}
__global__ __launch_bounds__(256) void dw_router_reduce_kernel(int64_t n, int nch,
                                                               const float* __restrict__ part,
                                                               float* __restrict__ dw) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float acc = 0.f;
    int c = 0;
    for (; c + 8 <= nch; c += 8) {  // 8 loads in flight, added in chunk order
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = part[(int64_t)(c + q) * n + i];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc += v[q];
    }
    for (; c < nch; ++c) acc += part[(int64_t)c * n + i];
    dw[i] = acc;
  }
}

// ---- operands of the K-grouped weight-gradient products ----------------------------------------
// dW_e = A_e^T B_e over expert e's kept rows. The 256 x 256 kernel's K-grouped mode takes A_e^T
// stored K-contiguous: the experts' transposed operands side by side in one (M, lda) matrix,
// expert e in columns kg_off[e] .. kg_off[e + 1] (its kept-row count rounded up to a multiple
// of 128, at least 128), zero past its own rows. B_e is read in place: rows offsets[e] ..
// offsets[e] + (kg_off[e + 1] - kg_off[e]) of the compact (rows, N) buffer, the rows past the
// expert's own multiplying those zeros (so they must be finite: the 128 rows after the last
// kept row are cleared).
constexpr int kKgAlign = 128;

// kg_off (E + 1) from the compact offsets, and the group row offsets e * M1 and e * M2.
__global__ __launch_bounds__(256) void kg_prep_kernel(int E, const int32_t* __restrict__ offsets,
                                                      int64_t M1, int64_t M2,
                                                      int32_t* __restrict__ kg_off,
                                                      int32_t* __restrict__ grow1,
                                                      int32_t* __restrict__ grow2) {
  for (int e = threadIdx.x; e <= E; e += 256) {
    grow1[e] = (int32_t)(e * M1);
    grow2[e] = (int32_t)(e * M2);
  }
  if (threadIdx.x == 0) {
    int32_t acc = 0;
    for (int e = 0; e < E; ++e) {
      kg_off[e] = acc;
      const int32_t n = offsets[e + 1] - offsets[e];
      acc += n <= 0 ? kKgAlign : (n + kKgAlign - 1) / kKgAlign * kKgAlign;
    }
    kg_off[E] = acc;
  }
}

// kg_map[j] = the compact row of column j of the transposed operand, or -1 (a zero column).
__global__ __launch_bounds__(256) void kg_map_kernel(int64_t ncols, int E,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ kg_off,
                                                     int32_t* __restrict__ kg_map) {
  const int32_t total = kg_off[E];
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < ncols;
       j += (int64_t)gridDim.x * 256) {
    int32_t r = -1;
    if (j < total) {
      int lo = 0, hi = E - 1;  // the last e with kg_off[e] <= j
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (kg_off[mid] <= j) lo = mid;
        else hi = mid - 1;
      }
      const int32_t i = (int32_t)j - kg_off[lo];
      if (i < offsets[lo + 1] - offsets[lo]) r = offsets[lo] + i;
    }
    kg_map[j] = r;
  }
}

// AT[m, j] = src[row(j), m] (row(j) = kg_map[j], through gather[.] / gather_div when given;
// zero for kg_map[j] < 0), for the columns j < kg_off[E]. 64 x 64 tiles through LDS; bf16,
// M % 8 == 0.
__global__ __launch_bounds__(256) void kg_transpose_kernel(int64_t M, int64_t lda, int E,
                                                           const int32_t* __restrict__ kg_off,
                                                           const int32_t* __restrict__ kg_map,
                                                           const uint16_t* __restrict__ src,
                                                           const int32_t* __restrict__ gather,
                                                           int gather_div,
                                                           uint16_t* __restrict__ at) {
  __shared__ __align__(16) uint16_t tile[64][64 + 8];
  const int64_t j0 = (int64_t)blockIdx.x * 64, m0 = (int64_t)blockIdx.y * 64;
  if (j0 >= kg_off[E]) return;  // kg_off[E] is a multiple of 128: tiles are all in or all out
  const int t = threadIdx.x;
  {
    const int jj = t >> 2, mc = (t & 3) * 16;
    const int32_t r = kg_map[j0 + jj];
    const int64_t srow = r < 0 ? -1 : (gather ? gather[r] / gather_div : r);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t m = m0 + mc + 8 * h;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (srow >= 0 && m < M) v = *(const uint4*)(src + srow * M + m);
      *(uint4*)&tile[jj][mc + 8 * h] = v;
    }
  }
  __syncthreads();
  const int mm = t >> 2, jc = (t & 3) * 16;
  if (m0 + mm >= M) return;
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = (uint32_t)tile[jc + 2 * i][mm] | ((uint32_t)tile[jc + 2 * i + 1][mm] << 16);
  uint4* dst = (uint4*)(at + (m0 + mm) * lda + j0 + jc);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// Clear rows offsets[E] .. + kKgAlign of a (rows, N) bf16 buffer (N % 8 == 0).
__global__ __launch_bounds__(256) void kg_clear_tail_kernel(int E, const int32_t* __restrict__ offsets,
                                                            int64_t N, uint16_t* __restrict__ buf) {
  const int64_t base = (int64_t)offsets[E] * N, n8 = (int64_t)kKgAlign * N / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256)
    *(uint4*)(buf + base + 8 * i) = make_uint4(0u, 0u, 0u, 0u);
}

// dx[t] = sum over the token's kept slots of the dx rows (dxr1, plus dxr2 when non-null;
// float32 sums, ascending j) plus sum_e dl[t, e] W_router[:, e]; one wave per token.
template <typename TIn, typename TR>
__global__ __launch_bounds__(kThreads) void dx_kernel(int64_t T, int64_t D, int E, int k,
                                                      const TR* __restrict__ dxr1,
                                                      const TR* __restrict__ dxr2,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ dl,
                                                      const TIn* __restrict__ w_router,
                                                      TIn* __restrict__ dx) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + wave_id();
  if (t >= T) return;
  for (int64_t c = lane; c < D; c += kWave) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int row = slot_row[t * k + j];
      if (row >= 0) {
        acc += load_as_f32(dxr1, (int64_t)row * D + c);
        if (dxr2) acc += load_as_f32(dxr2, (int64_t)row * D + c);
      }
    }
    for (int e = 0; e < E; ++e) acc = fmaf(dl[t * E + e], load_as_f32(w_router, c * E + e), acc);
    store_from_f32(dx, t * D + c, acc);
  }
}

// bf16 versions of the three kernels above, 8 elements a lane (16-byte loads and stores), for
// DH % 8 == 0 (activations) and D % 8 == 0, E % 8 == 0 (dx). Same arithmetic, same order.

__global__ __launch_bounds__(256) void act_backward_bf16x8_kernel(
    int64_t DH, int kind, const int32_t* __restrict__ offsets, int E, const uint4* __restrict__ a,
    const uint4* __restrict__ b, const uint4* __restrict__ dh, uint4* __restrict__ da,
    uint4* __restrict__ db) {
  const int64_t n = (int64_t)offsets[E] * DH / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    float av[8], g[8], ra[8];
    unpack8(a[i], av);
    unpack8(dh[i], g);
    if (kind == MOE_EXPERT_SWIGLU) {
      float bv[8], rb[8];
      unpack8(b[i], bv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float sg = 1.f / (1.f + __expf(-av[q]));
        ra[q] = g[q] * bv[q] * sg * (1.f + av[q] * (1.f - sg));
        rb[q] = g[q] * av[q] * sg;
      }
      db[i] = pack8(rb);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) ra[q] = av[q] > 0.f ? g[q] : 0.f;
    }
    da[i] = pack8(ra);
  }
}

// One wave per token; lane l handles columns 8 (l + 64 i) .. + 7.
__global__ __launch_bounds__(kThreads) void dx_bf16x8_kernel(int64_t T, int64_t D, int E, int k,
                                                             const uint16_t* __restrict__ dxr1,
                                                             const uint16_t* __restrict__ dxr2,
                                                             const int32_t* __restrict__ slot_row,
                                                             const float* __restrict__ dl,
                                                             const uint16_t* __restrict__ w_router,
                                                             uint16_t* __restrict__ dx) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + wave_id();
  if (t >= T) return;
  for (int64_t c = 8 * lane; c < D; c += 8 * kWave) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int row = slot_row[t * k + j];
      if (row >= 0) {
        float v[8];
        unpack8(*(const uint4*)(dxr1 + (int64_t)row * D + c), v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += v[q];
        if (dxr2) {
          unpack8(*(const uint4*)(dxr2 + (int64_t)row * D + c), v);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] += v[q];
        }
      }
    }
    for (int e0 = 0; e0 < E; e0 += 8) {
      float d8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) d8[i] = dl[t * E + e0 + i];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float w[8];
        unpack8(*(const uint4*)(w_router + (c + q) * E + e0), w);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[q] = fmaf(d8[i], w[i], acc[q]);
      }
    }
    *(uint4*)(dx + t * D + c) = pack8(acc);
  }
}

size_t a256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

// ---- scratch layout and the launch sequence ----------------------------------------------------

struct BwdLayout {
  size_t route, idx, gates, logits, aux, counts, offsets, perm, slot_row, blkc, lrank;
  size_t a, b, h, y, dy, dh, da, db, dxr, dgates, dl, gsplit, gctr;
  size_t dwr_part, kg_off, kg_grow1, kg_grow2, kg_map, kg_at;
  int dwr_chunks;
  int64_t dwr_tc, kg_lda;
  bool kg;
  size_t total;
};

// Token chunks of the router-weight gradient's first level.
// Token chunks of 32 (more, longer ones when the partials, chunks x D x E floats, would pass
// 64 MB), at most 256.
static int dwr_chunks_of(const Problem& q) {
  int64_t n = (q.T + 31) / 32;
  const int64_t per = std::max<int64_t>(1, (int64_t)q.D * q.E * 4);
  n = std::min<int64_t>(n, std::max<int64_t>(1, ((int64_t)64 << 20) / per));
  return (int)std::max<int64_t>(1, std::min<int64_t>(n, 256));
}

static BwdLayout bwd_layout(const Problem& q) {
  BwdLayout L;
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off = a256(off + n);
    return o;
  };
  const size_t es = q.dtype == MOE_BF16 ? 2 : 4;
  const size_t R = (size_t)q.slots(), T = (size_t)q.T, E = (size_t)q.E;
  const size_t DH = (size_t)(q.kind == MOE_EXPERT_LINEAR ? 0 : q.DH);
  L.route = take(route_ws_bytes(q));
  L.idx = take(R * 4);
  L.gates = take(R * 4);
  L.logits = take(T * E * 4);
  L.aux = take(4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take(R * 4);
  L.slot_row = take(R * 4);
  L.blkc = take((size_t)dispatch_blocks(q) * E * 4);
  L.lrank = take(R * 4);
  L.a = take(R * DH * es);
  L.b = take(q.kind == MOE_EXPERT_SWIGLU ? R * DH * es : 0);
  L.h = take(R * DH * es);
  L.y = take(R * (size_t)q.D_out * es);
  // the K-grouped weight gradients (bf16): B operands get kKgAlign spare rows
  const int64_t Mmax = std::max<int64_t>(q.D, q.kind == MOE_EXPERT_LINEAR ? 0 : q.DH);
  L.kg = q.dtype == MOE_BF16 && q.T > 0 && q.D % 8 == 0 && q.D_out % 8 == 0 &&
         (q.kind == MOE_EXPERT_LINEAR || q.DH % 8 == 0) &&
         (int64_t)q.E * (Mmax + 1) < ((int64_t)1 << 31) &&
         (int64_t)R + (int64_t)kKgAlign * (E + 1) < ((int64_t)1 << 31);
  const size_t spare = L.kg ? kKgAlign : 0;
  L.kg_lda = L.kg ? ((int64_t)R + kKgAlign * (int64_t)E + kKgAlign - 1) / kKgAlign * kKgAlign : 0;
  L.dy = take((R + spare) * (size_t)q.D_out * es);
  L.dh = take(R * DH * es);
  L.da = take((R + spare) * DH * es);
  L.db = take(q.kind == MOE_EXPERT_SWIGLU ? (R + spare) * DH * es : 0);
  L.dxr = take(R * (size_t)q.D * 4);
  L.dgates = take(R * 4);
  L.dl = take(T * E * 4);
  const bool split = q.dtype == MOE_BF16 && q.T > 0;
  L.gsplit = take(split ? (size_t)kSplitSlots * kSplitSlotFloats * sizeof(float) : 0);
  L.gctr = take(split ? (size_t)(kSplitSlots + kQueueInts) * sizeof(int32_t) : 0);
  L.dwr_chunks = dwr_chunks_of(q);
  L.dwr_tc = (q.T + L.dwr_chunks - 1) / L.dwr_chunks;
  L.dwr_part = take((size_t)L.dwr_chunks * (size_t)q.D * E * 4);
  L.kg_off = take(L.kg ? (E + 1) * 4 : 0);
  L.kg_grow1 = take(L.kg ? (E + 1) * 4 : 0);
  L.kg_grow2 = take(L.kg ? (E + 1) * 4 : 0);
  L.kg_map = take(L.kg ? (size_t)L.kg_lda * 4 : 0);
  L.kg_at = take(L.kg ? (size_t)Mmax * (size_t)L.kg_lda * 2 : 0);
  L.total = off;
  return L;
}

size_t backward_ws_bytes(const Problem& q) { return bwd_layout(q).total; }

SavedLayout saved_layout(const Problem& q) {
  SavedLayout S;
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off = a256(off + n);
    return o;
  };
  const size_t es = q.dtype == MOE_BF16 ? 2 : 4;
  const size_t R = (size_t)q.slots();
  const size_t DH = (size_t)(q.kind == MOE_EXPERT_LINEAR ? 0 : q.DH);
  S.logits = take((size_t)q.T * q.E * 4);
  S.perm = take(R * 4);
  S.a = take(R * DH * es);
  S.b = take(q.kind == MOE_EXPERT_SWIGLU ? R * DH * es : 0);
  S.h = take(R * DH * es);
  S.y = take(R * (size_t)q.D_out * es);
  S.total = off;
  return S;
}

namespace {

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

struct GemmRes {
  float* split_ws;
  int32_t* split_ctr;
  int32_t* queue;
  int ncu;
};

hipError_t nt(const Problem& q, const void* A0, const void* A1, const void* W0, const void* W1,
              int64_t K, int64_t N, const int32_t* offsets, void* C, bool c_f32, hipStream_t s,
              const GemmRes& res, const int32_t* a_gather = nullptr) {
  if (a_gather && !(q.dtype == MOE_BF16 && !A1 && !c_f32 && K % 128 == 0 && res.queue))
    return hipErrorInvalidValue;  // only the 256 x 256 path gathers A's rows
  if (q.dtype == MOE_BF16 && !A1 && !c_f32 && K % 128 == 0 && res.queue) {
    // the forward's 256 x 256 pipeline, reading the weight K-major
    GroupedGemm f{};
    f.A = A0;
    f.lda = K;
    f.a_gather = a_gather;  // row r reads A row a_gather[r] / top_k (a token's row)
    f.gather_div = a_gather ? q.top_k : 1;
    f.B0 = W0;
    f.B1 = nullptr;
    f.C = C;
    f.offsets = offsets;
    f.E = q.E;
    f.K = K;
    f.N = N;
    f.max_rows = q.slots();
    f.epilogue = EPI_NONE;
    f.dtype = q.dtype;
    f.split_ws = res.split_ws;
    f.split_slots = kSplitSlots;
    f.split_ctr = res.split_ctr;
    f.queue = res.queue;
    f.ncu = res.ncu;
    f.b_kmajor = true;
    return launch_grouped_gemm(f, s);
  }
  BwdGemm g{};
  g.A0 = A0;
  g.A1 = A1;
  g.W0 = W0;
  g.W1 = W1;
  g.offsets = offsets;
  g.E = q.E;
  g.K = K;
  g.N = N;
  g.lda = K;
  g.C = C;
  g.max_rows = q.slots();
  if (q.dtype == MOE_BF16) {
    const dim3 grid((unsigned)((g.max_rows + kBM - 1) / kBM + q.E), (unsigned)((N + kBN - 1) / kBN));
    if (A1 && c_f32) hipLaunchKernelGGL((nt_bf16_kernel<2, float>), grid, dim3(kThreads), 0, s, g);
    else if (A1) hipLaunchKernelGGL((nt_bf16_kernel<2, uint16_t>), grid, dim3(kThreads), 0, s, g);
    else if (c_f32) hipLaunchKernelGGL((nt_bf16_kernel<1, float>), grid, dim3(kThreads), 0, s, g);
    else hipLaunchKernelGGL((nt_bf16_kernel<1, uint16_t>), grid, dim3(kThreads), 0, s, g);
  } else {
    const dim3 grid((unsigned)((g.max_rows + 15) / 16 + q.E), (unsigned)((N + 15) / 16));
    if (A1) hipLaunchKernelGGL(nt_f32_kernel<2>, grid, dim3(kThreads), 0, s, g);
    else hipLaunchKernelGGL(nt_f32_kernel<1>, grid, dim3(kThreads), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t tn(const Problem& q, const void* A, int64_t lda, const int32_t* gather, int gather_div,
              const void* B, int64_t M, int64_t N, const int32_t* offsets, void* C, hipStream_t s) {
  BwdGemm g{};
  g.A0 = A;
  g.lda = lda;
  g.gather = gather;
  g.gather_div = gather_div;
  g.B = B;
  g.M = M;
  g.N = N;
  g.offsets = offsets;
  g.E = q.E;
  g.C = C;
  if (q.dtype == MOE_BF16) {
    const dim3 grid((unsigned)((M + kBM - 1) / kBM), (unsigned)((N + kBN - 1) / kBN), (unsigned)q.E);
    hipLaunchKernelGGL(tn_bf16_kernel<uint16_t>, grid, dim3(kThreads), 0, s, g);
  } else {
    const dim3 grid((unsigned)((M + 15) / 16), (unsigned)((N + 15) / 16), (unsigned)q.E);
    hipLaunchKernelGGL(tn_f32_kernel, grid, dim3(kThreads), 0, s, g);
  }
  return hipGetLastError();
}

// Weight gradient dW_e = A_e^T B_e through the K-grouped 256 x 256 kernel: kg_transpose
// writes the transposed operand (src's kept rows, (rows, M), gathered when `gather`), kg_gemm
// multiplies it with B; tn_kg does both.
hipError_t kg_transpose(const Problem& q, const BwdLayout& L, void* ws, const void* src,
                        const int32_t* gather, int gather_div, int64_t M, hipStream_t s) {
  const dim3 tgrid((unsigned)(L.kg_lda / 64), (unsigned)((M + 63) / 64));
  hipLaunchKernelGGL(kg_transpose_kernel, tgrid, dim3(256), 0, s, M, L.kg_lda, q.E,
                     (const int32_t*)at<int32_t>(ws, L.kg_off),
                     (const int32_t*)at<int32_t>(ws, L.kg_map), (const uint16_t*)src, gather,
                     gather_div, at<uint16_t>(ws, L.kg_at));
  return hipGetLastError();
}

hipError_t kg_gemm(const Problem& q, const BwdLayout& L, void* ws, int64_t M,
                   const int32_t* grow, const void* B, int64_t N, const int32_t* offsets, void* C,
                   const GemmRes& res, hipStream_t s) {
  GroupedGemm f{};
  f.A = at<uint16_t>(ws, L.kg_at);
  f.lda = L.kg_lda;
  f.a_gather = nullptr;
  f.gather_div = 1;
  f.B0 = B;
  f.B1 = nullptr;
  f.C = C;
  f.offsets = grow;
  f.E = q.E;
  f.K = kKgAlign;
  f.N = N;
  f.max_rows = (int64_t)q.E * M;
  f.epilogue = EPI_NONE;
  f.dtype = q.dtype;
  f.split_ws = nullptr;
  f.split_ctr = nullptr;
  f.queue = res.queue;
  f.ncu = res.ncu;
  f.k_grouped = true;
  f.k_offsets = at<int32_t>(ws, L.kg_off);
  f.b_offsets = offsets;
  f.group_rows = M;
  return launch_grouped_gemm(f, s);
}

hipError_t tn_kg(const Problem& q, const BwdLayout& L, void* ws, const void* src,
                 const int32_t* gather, int gather_div, int64_t M, const int32_t* grow,
                 const void* B, int64_t N, const int32_t* offsets, void* C, const GemmRes& res,
                 hipStream_t s) {
  hipError_t err = kg_transpose(q, L, ws, src, gather, gather_div, M, s);
  return err == hipSuccess ? kg_gemm(q, L, ws, M, grow, B, N, offsets, C, res, s) : err;
}

// The forward GEMM A_rows -> C without an epilogue (to recompute pre-activations / outputs).
hipError_t fwd_gemm(const Problem& q, const void* A, int64_t lda, const int32_t* gather,
                    const void* W, int64_t K, int64_t N, const int32_t* offsets, void* C,
                    float* split_ws, int64_t split_slots, int32_t* split_ctr, int32_t* queue,
                    int ncu, hipStream_t s) {
  GroupedGemm g{};
  g.A = A;
  g.lda = lda;
  g.a_gather = gather;
  g.gather_div = q.top_k;
  g.B0 = W;
  g.B1 = nullptr;
  g.C = C;
  g.offsets = offsets;
  g.E = q.E;
  g.K = K;
  g.N = N;
  g.max_rows = q.slots();
  g.epilogue = EPI_NONE;
  g.dtype = q.dtype;
  g.split_ws = split_ws;
  g.split_slots = split_slots;
  g.split_ctr = split_ctr;
  g.ncu = ncu;
  g.queue = queue;
  return launch_grouped_gemm(g, s);
}

// The forward quantities the backward needs, by pointer: from the recompute inside
// moe_backward, or from a training forward's saved state.
struct BwdInputs {
  const int32_t* idx;
  const float* gates;
  const float* logits;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* slot_row;
  const void* a;
  const void* b;
  const void* h;
  const void* y;
};

hipError_t backward_from(const Problem& q, const BwdInputs& in, const void* x,
                         const void* w_router, const void* w1, const void* w3, const void* w2,
                         const void* dout, float d_aux, void* dx, float* dw_router, float* dbias,
                         void* dw1, void* dw3, void* dw2, void* ws, bool tickets_zeroed,
                         hipStream_t s);

// bf16 ReLU / SwiGLU layers whose dgrad runs on the 256 x 256 path take the gate gradient
// from h and g = dout W2^T (act_backward_rows) instead of from y, so they need no y.
bool dgate_from_h(const Problem& q, const void* dout) {
  return q.dtype == MOE_BF16 && q.kind != MOE_EXPERT_LINEAR && q.T > 0 && q.D_out % 128 == 0 &&
         q.DH % 8 == 0 && (uintptr_t)dout % 16 == 0;
}

}  // namespace

hipError_t run_experts_saving(const Problem& q, const void* x, const int32_t* perm,
                              const int32_t* offsets, const void* w1, const void* w3,
                              const void* w2, void* a, void* b, void* h, void* y,
                              float* split_ws, int64_t split_slots, int32_t* split_ctr,
                              int32_t* queue, int ncu, hipStream_t s) {
  const int64_t D = q.D, DH = q.DH, Do = q.D_out;
  if (q.kind == MOE_EXPERT_LINEAR)
    return fwd_gemm(q, x, D, perm, w1, D, Do, offsets, y, split_ws, split_slots, split_ctr, queue, ncu, s);
  const bool swiglu = q.kind == MOE_EXPERT_SWIGLU;
  GroupedGemm g{};
  g.A = x;
  g.lda = D;
  g.a_gather = perm;
  g.gather_div = q.top_k;
  g.B0 = w1;
  g.B1 = swiglu ? w3 : nullptr;
  g.C = h;
  g.offsets = offsets;
  g.E = q.E;
  g.K = D;
  g.N = DH;
  g.max_rows = q.slots();
  g.epilogue = swiglu ? EPI_SWIGLU : EPI_RELU;
  g.dtype = q.dtype;
  g.split_ws = split_ws;
  g.split_slots = split_slots;
  g.split_ctr = split_ctr;
  g.ncu = ncu;
  g.queue = queue;
  // the 256 x 256 kernel stores the pre-activations beside h; elsewhere they take products of
  // their own (the same accumulation, so the same values)
  const bool saving = q.dtype == MOE_BF16 && D % 128 == 0 && queue != nullptr;
  if (saving) {
    g.pre_a = a;
    g.pre_b = swiglu ? b : nullptr;
  }
  hipError_t err = launch_grouped_gemm(g, s);
  if (!saving) {
    if (err == hipSuccess)
      err = fwd_gemm(q, x, D, perm, w1, D, DH, offsets, a, split_ws, split_slots, split_ctr, queue, ncu, s);
    if (err == hipSuccess && swiglu)
      err = fwd_gemm(q, x, D, perm, w3, D, DH, offsets, b, split_ws, split_slots, split_ctr, queue, ncu, s);
  }
  if (err == hipSuccess && y)  // (the backward of a bf16 layer does without y: dgate_from_h)
    err = fwd_gemm(q, h, DH, nullptr, w2, DH, Do, offsets, y, split_ws, split_slots, split_ctr, queue, ncu, s);
  return err;
}

hipError_t launch_backward(const Problem& q, const void* x, const void* w_router, const float* bias,
                           const void* w1, const void* w3, const void* w2, const void* dout,
                           float d_aux, void* dx, float* dw_router, float* dbias, void* dw1,
                           void* dw3, void* dw2, void* ws, hipStream_t s) {
  const BwdLayout L = bwd_layout(q);
  const bool bf16 = q.dtype == MOE_BF16;
  int32_t* idx = at<int32_t>(ws, L.idx);
  float* gates = at<float>(ws, L.gates);
  float* logits = at<float>(ws, L.logits);
  int32_t* counts = at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* perm = at<int32_t>(ws, L.perm);
  int32_t* slot_row = at<int32_t>(ws, L.slot_row);
  // 1. decisions, gates and logits, exactly as the forward takes them
  bool dispatched = false;
  hipError_t err = launch_route_full(q, x, w_router, bias, RouteOpts{}, idx, gates, logits,
                                     nullptr, at<float>(ws, L.aux), counts, nullptr,
                                     at<void>(ws, L.route), s, offsets, &dispatched);
  // 2. dispatch (counts, offsets, permutation, slot rows); it also clears the GEMMs' split
  //    tickets and work queue
  int32_t* tickets = (bf16 && q.T > 0) ? at<int32_t>(ws, L.gctr) : nullptr;
  if (err == hipSuccess && dispatched)
    err = launch_place_after_route(q, idx, at<void>(ws, L.route), at<float>(ws, L.aux), counts,
                                   nullptr, offsets, perm, slot_row, s, tickets,
                                   tickets ? kSplitSlots + kQueueInts : 0);
  else if (err == hipSuccess)
    err = launch_dispatch(q, idx, x, counts, offsets, perm, slot_row, nullptr,
                          at<int32_t>(ws, L.blkc), at<int32_t>(ws, L.lrank), s, tickets,
                          tickets ? kSplitSlots + kQueueInts : 0);
  if (q.T == 0 || err != hipSuccess) return err;
  // 3. the experts' forward quantities on the kept rows, as a training forward keeps them
  const int ncu = bf16 ? device_split_cus() : 0;
  int32_t* queue = tickets ? tickets + kSplitSlots : nullptr;
  err = run_experts_saving(q, x, perm, offsets, w1, w3, w2, at<void>(ws, L.a), at<void>(ws, L.b),
                           at<void>(ws, L.h), dgate_from_h(q, dout) ? nullptr : at<void>(ws, L.y),
                           (tickets && ncu > 0) ? at<float>(ws, L.gsplit) : nullptr, kSplitSlots,
                           (tickets && ncu > 0) ? tickets : nullptr, queue, ncu, s);
  if (err != hipSuccess) return err;
  const BwdInputs in{idx, gates, logits, counts, offsets, perm, slot_row,
                     at<void>(ws, L.a), at<void>(ws, L.b), at<void>(ws, L.h), at<void>(ws, L.y)};
  return backward_from(q, in, x, w_router, w1, w3, w2, dout, d_aux, dx, dw_router, dbias, dw1,
                       dw3, dw2, ws, true, s);
}

hipError_t launch_backward_saved(const Problem& q, const int32_t* idx, const float* gates,
                                 const int32_t* counts, const int32_t* offsets,
                                 const int32_t* slot_row, const void* saved, const void* x,
                                 const void* w_router, const void* w1, const void* w3,
                                 const void* w2, const void* dout, float d_aux, void* dx,
                                 float* dw_router, float* dbias, void* dw1, void* dw3, void* dw2,
                                 void* ws, hipStream_t s) {
  if (q.T == 0) return hipSuccess;
  const SavedLayout S = saved_layout(q);
  const char* sv = (const char*)saved;
  const BwdInputs in{idx, gates, (const float*)(sv + S.logits), counts, offsets,
                     (const int32_t*)(sv + S.perm), slot_row, sv + S.a, sv + S.b, sv + S.h,
                     sv + S.y};
  return backward_from(q, in, x, w_router, w1, w3, w2, dout, d_aux, dx, dw_router, dbias, dw1,
                       dw3, dw2, ws, false, s);
}

namespace {

hipError_t backward_from(const Problem& q, const BwdInputs& in, const void* x,
                         const void* w_router, const void* w1, const void* w3, const void* w2,
                         const void* dout, float d_aux, void* dx, float* dw_router, float* dbias,
                         void* dw1, void* dw3, void* dw2, void* ws, bool tickets_zeroed,
                         hipStream_t s) {
  const BwdLayout L = bwd_layout(q);
  const bool bf16 = q.dtype == MOE_BF16;
  const bool linear = q.kind == MOE_EXPERT_LINEAR, swiglu = q.kind == MOE_EXPERT_SWIGLU;
  const int32_t* idx = in.idx;
  const float* gates = in.gates;
  const float* logits = in.logits;
  const int32_t* counts = in.counts;
  const int32_t* offsets = in.offsets;
  const int32_t* perm = in.perm;
  const int32_t* slot_row = in.slot_row;
  hipError_t err = hipSuccess;
  float* split_ws = nullptr;
  int32_t* split_ctr = nullptr;
  int32_t* queue = nullptr;
  const int ncu = bf16 ? device_split_cus() : 0;
  if (bf16 && q.T > 0) {
    int32_t* ctr = at<int32_t>(ws, L.gctr);
    queue = ctr + kSplitSlots;
    if (ncu > 0) {
      split_ws = at<float>(ws, L.gsplit);
      split_ctr = ctr;
    }
  }
  const GemmRes res{split_ws, split_ctr, queue, ncu};
  if (q.T == 0) return hipSuccess;  // nothing routed: the caller's outputs are left as they are
  // the GEMMs' split tickets and work queue start at zero (the recompute's dispatch cleared
  // them; a saved forward's workspace is another buffer)
  if (queue && !tickets_zeroed) err = launch_zero_tickets(at<int32_t>(ws, L.gctr), kSplitSlots + kQueueInts, s);
  const int64_t D = q.D, DH = q.DH, Do = q.D_out;
  const void* a = in.a;
  const void* b = in.b;
  const void* h = in.h;
  const void* y = in.y;
  void* dy = at<void>(ws, L.dy);
  void* dh = at<void>(ws, L.dh);
  void* da = at<void>(ws, L.da);
  void* db = at<void>(ws, L.db);
  // dx rows: float32 for float32 layers (both halves in one product); two bf16 halves
  // (da W1^T and db W3^T) for bf16 layers, added in the dx kernel
  float* dxr = at<float>(ws, L.dxr);
  uint16_t* dxr1 = at<uint16_t>(ws, L.dxr);
  uint16_t* dxr2 = dxr1 + (size_t)q.slots() * q.D;
  float* dgates = at<float>(ws, L.dgates);
  float* dl = at<float>(ws, L.dl);
  // elementwise kernels: about two 8-element vectors a thread over the worst-case rows
  const unsigned ew_grid = (unsigned)std::max<int64_t>(
      1, std::min<int64_t>(((int64_t)q.slots() * std::max<int64_t>(q.DH, 8) / 8 + 511) / 512,
                           65536));
  // K-grouped weight gradients: per-expert K ranges, group rows, the column map
  const bool kg = L.kg && queue != nullptr;
  int32_t* grow1 = at<int32_t>(ws, L.kg_grow1);  // e * D
  int32_t* grow2 = at<int32_t>(ws, L.kg_grow2);  // e * DH
  if (kg && err == hipSuccess) {
    hipLaunchKernelGGL(kg_prep_kernel, dim3(1), dim3(256), 0, s, q.E, (const int32_t*)offsets, D,
                       linear ? (int64_t)0 : DH, at<int32_t>(ws, L.kg_off), grow1, grow2);
    hipLaunchKernelGGL(kg_map_kernel, dim3((unsigned)std::min<int64_t>((L.kg_lda + 255) / 256, 4096)),
                       dim3(256), 0, s, L.kg_lda, q.E, (const int32_t*)offsets,
                       (const int32_t*)at<int32_t>(ws, L.kg_off), at<int32_t>(ws, L.kg_map));
    err = hipGetLastError();
  }
  auto clear_tail = [&](void* buf, int64_t N) {
    if (kg && err == hipSuccess) {
      hipLaunchKernelGGL(kg_clear_tail_kernel, dim3(64), dim3(256), 0, s, q.E,
                         (const int32_t*)offsets, N, (uint16_t*)buf);
      err = hipGetLastError();
    }
  };
  // 4. combine backward: dy rows and dgates (with dgate_from_h: dy rows here, kept slots'
  //    dgates in the activation backward)
  const bool from_h = dgate_from_h(q, dout) && queue != nullptr;
  if (err == hipSuccess && from_h) {
    hipLaunchKernelGGL(scale_dout_rows_bf16x8_kernel, dim3((unsigned)((q.T + 3) / 4)),
                       dim3(kThreads), 0, s, q.T, q.top_k, Do, (const uint16_t*)dout, slot_row,
                       gates, (uint16_t*)dy, dgates);
    err = hipGetLastError();
  } else if (err == hipSuccess) {
    const unsigned grid = (unsigned)((q.T + 3) / 4);
    if (bf16 && Do % 8 == 0 && (uintptr_t)dout % 16 == 0)
      hipLaunchKernelGGL(combine_backward_bf16x8_kernel, dim3(grid), dim3(kThreads), 0, s, q.T,
                         q.top_k, Do, (const uint16_t*)dout, (const uint16_t*)y, slot_row, gates,
                         (uint16_t*)dy, dgates);
    else if (bf16)
      hipLaunchKernelGGL(combine_backward_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, s, q.T,
                         q.top_k, Do, (const uint16_t*)dout, (const uint16_t*)y, slot_row, gates,
                         (uint16_t*)dy, dgates);
    else
      hipLaunchKernelGGL(combine_backward_kernel<float>, dim3(grid), dim3(kThreads), 0, s, q.T,
                         q.top_k, Do, (const float*)dout, (const float*)y, slot_row, gates,
                         (float*)dy, dgates);
    err = hipGetLastError();
  }
  // 5. experts backward
  clear_tail(dy, Do);
  if (linear) {
    if (err == hipSuccess)
      err = kg ? tn_kg(q, L, ws, x, perm, q.top_k, D, grow1, dy, Do, offsets, dw1, res, s)
               : tn(q, x, D, perm, q.top_k, dy, D, Do, offsets, dw1, s);
    if (err == hipSuccess)
      err = bf16 ? nt(q, dy, nullptr, w1, nullptr, Do, D, offsets, dxr1, false, s, res)
                 : nt(q, dy, nullptr, w1, nullptr, Do, D, offsets, dxr, true, s, res);
  } else {
    // dh = dy W2^T; with from_h, g = dout W2^T over the slots' token rows (the gate is applied
    // in the activation backward)
    if (err == hipSuccess)
      err = from_h ? nt(q, dout, nullptr, w2, nullptr, Do, DH, offsets, dh, false, s, res, perm)
                   : nt(q, dy, nullptr, w2, nullptr, Do, DH, offsets, dh, false, s, res);
    if (err == hipSuccess)
      err = kg ? tn_kg(q, L, ws, h, nullptr, 1, DH, grow2, dy, Do, offsets, dw2, res, s)
               : tn(q, h, DH, nullptr, 1, dy, DH, Do, offsets, dw2, s);
    if (err == hipSuccess && from_h) {
      hipLaunchKernelGGL(act_backward_rows_bf16x8_kernel,
                         dim3((unsigned)((q.slots() + kThreads / kWave - 1) / (kThreads / kWave))),
                         dim3(kThreads), 0, s, DH, q.kind, offsets, q.E, perm, gates,
                         (const uint16_t*)a, (const uint16_t*)b, (const uint16_t*)dh,
                         (uint16_t*)da, (uint16_t*)db, dgates);
      err = hipGetLastError();
    } else if (err == hipSuccess) {
      if (bf16 && DH % 8 == 0)
        hipLaunchKernelGGL(act_backward_bf16x8_kernel, dim3(ew_grid), dim3(256), 0, s, DH, q.kind,
                           offsets, q.E, (const uint4*)a, (const uint4*)b, (const uint4*)dh,
                           (uint4*)da, (uint4*)db);
      else if (bf16)
        hipLaunchKernelGGL(act_backward_kernel<uint16_t>, dim3(ew_grid), dim3(256), 0, s, DH,
                           q.kind, offsets, q.E, (const uint16_t*)a, (const uint16_t*)b,
                           (const uint16_t*)dh, (uint16_t*)da, (uint16_t*)db);
      else
        hipLaunchKernelGGL(act_backward_kernel<float>, dim3(ew_grid), dim3(256), 0, s, DH, q.kind,
                           offsets, q.E, (const float*)a, (const float*)b, (const float*)dh,
                           (float*)da, (float*)db);
      err = hipGetLastError();
    }
    clear_tail(da, DH);
    if (swiglu) clear_tail(db, DH);
    if (kg) {
      // one transposed operand (the gathered x) for both products
      if (err == hipSuccess)
        err = tn_kg(q, L, ws, x, perm, q.top_k, D, grow1, da, DH, offsets, dw1, res, s);
      if (err == hipSuccess && swiglu)
        err = kg_gemm(q, L, ws, D, grow1, db, DH, offsets, dw3, res, s);
    } else {
      if (err == hipSuccess) err = tn(q, x, D, perm, q.top_k, da, D, DH, offsets, dw1, s);
      if (err == hipSuccess && swiglu) err = tn(q, x, D, perm, q.top_k, db, D, DH, offsets, dw3, s);
    }
    if (bf16) {
      if (err == hipSuccess) err = nt(q, da, nullptr, w1, nullptr, DH, D, offsets, dxr1, false, s, res);
      if (err == hipSuccess && swiglu)
        err = nt(q, db, nullptr, w3, nullptr, DH, D, offsets, dxr2, false, s, res);
    } else if (err == hipSuccess) {
      err = nt(q, da, swiglu ? db : nullptr, w1, swiglu ? w3 : nullptr, DH, D, offsets, dxr, true,
               s, res);
    }
  }
  // 6. router backward, the router's gradients, and dx
  if (err == hipSuccess) {
    const unsigned grid = (unsigned)((q.T + 3) / 4);
    const int epl = (q.E + kWave - 1) / kWave;
    if (epl <= 1)
      hipLaunchKernelGGL(router_backward_kernel<1>, dim3(grid), dim3(kThreads), 0, s, q.T, q.E,
                         q.top_k, d_aux, logits, idx, gates, dgates, counts, dl);
    else if (epl <= 2)
      hipLaunchKernelGGL(router_backward_kernel<2>, dim3(grid), dim3(kThreads), 0, s, q.T, q.E,
                         q.top_k, d_aux, logits, idx, gates, dgates, counts, dl);
    else
      hipLaunchKernelGGL(router_backward_kernel<4>, dim3(grid), dim3(kThreads), 0, s, q.T, q.E,
                         q.top_k, d_aux, logits, idx, gates, dgates, counts, dl);
    if (dbias) hipLaunchKernelGGL(dbias_kernel, dim3(q.E), dim3(256), 0, s, q.T, q.E, dl, dbias);
    const dim3 wgrid((unsigned)((D + 255) / 256), (unsigned)((q.E + 7) / 8), (unsigned)L.dwr_chunks);
    float* part = at<float>(ws, L.dwr_part);
    const int64_t nw = D * q.E;
    const unsigned rgrid = (unsigned)std::min<int64_t>((nw + 255) / 256, 2048);
    if (bf16) {
      hipLaunchKernelGGL(dw_router_partial_kernel<uint16_t>, wgrid, dim3(256), 0, s, q.T, D, q.E,
                         L.dwr_tc, (const uint16_t*)x, dl, part);
      hipLaunchKernelGGL(dw_router_reduce_kernel, dim3(rgrid), dim3(256), 0, s, nw, L.dwr_chunks,
                         (const float*)part, dw_router);
      if (D % 8 == 0 && q.E % 8 == 0 && (uintptr_t)w_router % 16 == 0 && (uintptr_t)dx % 16 == 0)
        hipLaunchKernelGGL(dx_bf16x8_kernel, dim3(grid), dim3(kThreads), 0, s, q.T, D, q.E,
                           q.top_k, (const uint16_t*)dxr1,
                           (const uint16_t*)(swiglu ? dxr2 : nullptr), slot_row, dl,
                           (const uint16_t*)w_router, (uint16_t*)dx);
      else
        hipLaunchKernelGGL((dx_kernel<uint16_t, uint16_t>), dim3(grid), dim3(kThreads), 0, s, q.T,
                           D, q.E, q.top_k, (const uint16_t*)dxr1,
                           (const uint16_t*)(swiglu ? dxr2 : nullptr), slot_row, dl,
                           (const uint16_t*)w_router, (uint16_t*)dx);
    } else {
      hipLaunchKernelGGL(dw_router_partial_kernel<float>, wgrid, dim3(256), 0, s, q.T, D, q.E,
                         L.dwr_tc, (const float*)x, dl, part);
      hipLaunchKernelGGL(dw_router_reduce_kernel, dim3(rgrid), dim3(256), 0, s, nw, L.dwr_chunks,
                         (const float*)part, dw_router);
      hipLaunchKernelGGL((dx_kernel<float, float>), dim3(grid), dim3(kThreads), 0, s, q.T, D, q.E,
                         q.top_k, (const float*)dxr, (const float*)nullptr, slot_row, dl,
                         (const float*)w_router, (float*)dx);
    }
    err = hipGetLastError();
  }
  return err;
}

}  // namespace

}  // namespace moe

// Combine: out[t] = sum over kept slots j of gates[t, j] * y[slot_row[t*k + j]]
// (ML Grind "Mixture-of-Experts (MoE) Routing", Algorithm step 3 formula; a dropped slot
// adds nothing and the gates are not renormalised, as in the Sparsely-Gated Layer page's
// moe_forward). The inverse map slot_row lets one wave own one output row: it gathers the
// token's k expert rows with 16-byte loads and accumulates them in float32 in ascending j,
// so there are no atomics and the sum order is fixed.
#include <algorithm>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxWavesPerToken = 8;  // a wider row makes more than one pass a wave

__device__ __forceinline__ void unpack8(const uint4& u, float f[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint4 pack8(const float f[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// bf16 rows, N % 8 == 0, 16-byte aligned, top_k <= 64. A token's row is split into passes of
// U x 64 column chunks (16 bytes each), and wave w takes pass w % wpt of token w / wpt (wpt =
// 2^lw, the passes a row has rounded up, so a wave usually makes one pass). Lane j first loads slot j's row
// and gate, then a pass issues the KG x U 16-byte loads of KG slots and U column chunks per
// lane before any of them is used, so a wave has KG x U row loads in flight; the sum still runs
// over j ascending. With ONE (top_k <= KG) the token's slots are a single group, and each column
// chunk is summed, packed and stored as soon as its loads are in, so only the loads hold
// registers. (Passes spread over more waves beat longer passes: at the Mixtral shape, 4 waves
// of 2 chunks a lane per token took 18.5 us, 2 waves of 4 18.8-19.3 us, one wave of 8 20.4 us.)
template <int KG, int U, bool ONE, int LW>
__global__ __launch_bounds__(kThreads, 4) void combine_bf16x8_kernel(
    int64_t T, int k, int64_t n_vec, const uint4* __restrict__ y,
    const int32_t* __restrict__ slot_row, const float* __restrict__ gates,
    uint4* __restrict__ out) {
  const int gw = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWaves + wave_id()));
  constexpr int wpt = 1 << LW;
  const int64_t t = gw >> LW;
  const int pass = gw & (wpt - 1);
  if (t >= T) return;
  const int lane = lane_id();
  const int rl = lane < k ? slot_row[t * k + lane] : -1;
  const float gl = lane < k ? gates[t * k + lane] : 0.f;
  for (int64_t c0 = lane + (int64_t)pass * U * kWave; c0 < n_vec;
       c0 += (int64_t)wpt * U * kWave) {
    float acc[ONE ? 1 : U][8];
    if (!ONE) {
#pragma unroll
      for (int u = 0; u < (ONE ? 1 : U); ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
    }
    for (int j0 = 0; j0 < k; j0 += KG) {
      int r[KG];
      float g[KG];
      uint4 w[KG][U];
#pragma unroll
      for (int jj = 0; jj < KG; ++jj) {
        const int j = j0 + jj;
        r[jj] = j < k ? __builtin_amdgcn_readlane(rl, j) : -1;
        g[jj] = j < k ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                      __builtin_bit_cast(int, gl), j))
                      : 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t c = c0 + u * kWave;
          w[jj][u] = (r[jj] >= 0 && c < n_vec) ? y[(int64_t)r[jj] * n_vec + c]
                                               : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      if (ONE) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float a[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) a[i] = 0.f;
#pragma unroll
          for (int jj = 0; jj < KG; ++jj) {
            if (r[jj] < 0) continue;
            float v[8];
            unpack8(w[jj][u], v);
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] = fmaf(g[jj], v[i], a[i]);
          }
          const int64_t c = c0 + u * kWave;
          if (c < n_vec) out[t * n_vec + c] = pack8(a);
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < KG; ++jj) {
          if (r[jj] < 0) continue;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            float v[8];
            unpack8(w[jj][u], v);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[u][i] = fmaf(g[jj], v[i], acc[u][i]);
          }
        }
      }
    }
    if (!ONE) {
#pragma unroll
      for (int u = 0; u < (ONE ? 1 : U); ++u) {
        const int64_t c = c0 + u * kWave;
        if (c < n_vec) out[t * n_vec + c] = pack8(acc[u]);
      }
    }
  }
}

// Any element type and width: one element per lane step.
template <typename TE>
__global__ __launch_bounds__(kThreads) void combine_scalar_kernel(
    int64_t T, int k, int64_t N, const TE* __restrict__ y, const int32_t* __restrict__ slot_row,
    const float* __restrict__ gates, TE* __restrict__ out) {
  const int64_t t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWaves + wave_id()));
  if (t >= T) return;
  const int lane = lane_id();
  for (int64_t c = lane; c < N; c += kWave) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = slot_row[t * k + j];
      if (r < 0) continue;
      acc = fmaf(gates[t * k + j], load_as_f32(y, (int64_t)r * N + c), acc);
    }
    store_from_f32(out, t * N + c, acc);
  }
}

}  // namespace

hipError_t launch_combine(const Problem& p, const void* y, const int32_t* slot_row,
                          const float* gates, void* out, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const unsigned grid = (unsigned)((p.T + kWaves - 1) / kWaves);
  const bool al16 = ((uintptr_t)y % 16 == 0) && ((uintptr_t)out % 16 == 0);
  if (p.dtype == MOE_BF16 && p.D_out % 8 == 0 && al16 && p.top_k <= kWave) {
    // slots x column chunks of loads in flight per lane; a token's slots in one group when
    // top_k <= 8; a row's passes (U x 64 chunks each) on waves of their own
    const int64_t nv = p.D_out / 8;
    const uint4* yv = (const uint4*)y;
    uint4* ov = (uint4*)out;
#define MOE_COMBINE_LW(KG, U, ONE, LW)                                                       \
  hipLaunchKernelGGL((combine_bf16x8_kernel<KG, U, ONE, LW>), dim3(g2), dim3(kThreads), 0, s, \
                     p.T, p.top_k, nv, yv, slot_row, gates, ov)
#define MOE_COMBINE(KG, U, ONE)                                                              \
  do {                                                                                       \
    int lw = 0;                                                                              \
    while ((1 << lw) < kMaxWavesPerToken && ((int64_t)U * kWave << lw) < nv) ++lw;           \
    if ((p.T << lw) > INT32_MAX) lw = 0; /* wave ids are 32-bit */                           \
    const unsigned g2 = (unsigned)(((p.T << lw) + kWaves - 1) / kWaves);                     \
    switch (lw) {                                                                            \
      case 0: MOE_COMBINE_LW(KG, U, ONE, 0); break;                                          \
      case 1: MOE_COMBINE_LW(KG, U, ONE, 1); break;                                          \
      case 2: MOE_COMBINE_LW(KG, U, ONE, 2); break;                                          \
      default: MOE_COMBINE_LW(KG, U, ONE, 3); break;                                         \
    }                                                                                        \
  } while (0)
    if (p.top_k <= 2) {
      MOE_COMBINE(2, 2, true);
    } else if (p.top_k <= 4) {
      if (nv > 2 * kWave) MOE_COMBINE(4, 4, true);
      else MOE_COMBINE(4, 2, true);
    } else if (p.top_k <= 8) {
      MOE_COMBINE(8, 2, true);
    } else {
      MOE_COMBINE(8, 2, false);
    }
#undef MOE_COMBINE
#undef MOE_COMBINE_LW
  } else if (p.dtype == MOE_BF16) {
    hipLaunchKernelGGL(combine_scalar_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, s, p.T,
                       p.top_k, p.D_out, (const uint16_t*)y, slot_row, gates, (uint16_t*)out);
  } else {
    hipLaunchKernelGGL(combine_scalar_kernel<float>, dim3(grid), dim3(kThreads), 0, s, p.T,
                       p.top_k, p.D_out, (const float*)y, slot_row, gates, (float*)out);
  }
  return hipGetLastError();
}

}  // namespace moe

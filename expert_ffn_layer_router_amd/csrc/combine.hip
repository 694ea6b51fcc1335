// Combine: out[t] = sum over kept slots j of gates[t, j] * y[slot_row[t*k + j]]
// (ML Grind "Mixture-of-Experts (MoE) Routing", Algorithm step 3 formula; a dropped slot
// adds nothing and the gates are not renormalised, as in the Sparsely-Gated Layer page's
// moe_forward). The inverse map slot_row lets one wave own one output row: it gathers the
// token's k expert rows with 16-byte loads and accumulates them in float32 in ascending j,
// so there are no atomics and the sum order is fixed.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

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

// bf16 rows, N % 8 == 0, 16-byte aligned.
__global__ __launch_bounds__(kThreads) void combine_bf16x8_kernel(
    int64_t T, int k, int64_t n_vec, const uint4* __restrict__ y,
    const int32_t* __restrict__ slot_row, const float* __restrict__ gates,
    uint4* __restrict__ out) {
  const int64_t t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWaves + wave_id()));
  if (t >= T) return;
  const int lane = lane_id();
  // 4 column chunks a pass, so 4 k loads are in flight; each output is still the sum over
  // j ascending
  constexpr int U = 4;
  for (int64_t c0 = lane; c0 < n_vec; c0 += U * kWave) {
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = __builtin_amdgcn_readfirstlane(slot_row[t * k + j]);
      if (r < 0) continue;
      const float g = gates[t * k + j];
      uint4 w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * kWave;
        w[u] = c < n_vec ? y[(int64_t)r * n_vec + c] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float v[8];
        unpack8(w[u], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = fmaf(g, v[i], acc[u][i]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kWave;
      if (c < n_vec) out[t * n_vec + c] = pack8(acc[u]);
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
  if (p.dtype == MOE_BF16 && p.D_out % 8 == 0 && al16) {
    hipLaunchKernelGGL(combine_bf16x8_kernel, dim3(grid), dim3(kThreads), 0, s, p.T, p.top_k,
                       p.D_out / 8, (const uint4*)y, slot_row, gates, (uint4*)out);
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

// Dispatch: per-expert histogram, prefix-sum offsets, a stable permutation of the slots
// into expert-contiguous order, and the optional capacity with overflow dropped in token
// order. (ML Grind "Mixture-of-Experts (MoE) Routing", Algorithm step 3 and Follow-up;
// "Mixture of Experts: the Sparsely-Gated Layer", "Switch: top-1, one loss, and a rate
// limit" and its moe_forward: earlier tokens are kept before later ones.)
//
// Three kernels, all deterministic (no order-dependent atomics):
//  1. rank:  blocks of 256 tokens. Each wave builds, in LDS, one 64-bit lane mask per
//            expert (bit l set when the wave's token l chose that expert; integer OR is
//            order-independent). A slot's rank among the block's earlier tokens of its
//            expert is then a popcount of the lower lanes plus the earlier waves' counts.
//  2. scan:  one block. Per expert, an exclusive scan of the block counts in block order
//            (the rank base of each block), the total count, kept = min(count, capacity),
//            and the exclusive scan of kept over experts: the row offsets.
//  3. place: one wave per token. Rank = block base + local rank; kept iff rank < capacity;
//            row = offsets[e] + rank; perm[row] = slot, slot_row[slot] = row (or -1); the
//            token's x row is read once and written to each of its kept rows.
// Capacity-padded layout (Switch: every expert a fixed batch of `capacity` rows): place puts
// the slot at row e * capacity + rank instead, and a fourth kernel marks each batch's empty
// rows (perm = -1), zeroes them in the copy, and writes the batch starts e * capacity.
#include <algorithm>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
static_assert(kDispatchTokensPerBlock == kThreads, "one token per thread in the rank kernel");

__global__ __launch_bounds__(kThreads) void dispatch_rank_kernel(
    int64_t T, int k, int E, const int32_t* __restrict__ idx, int32_t* __restrict__ blk_counts,
    int32_t* __restrict__ local_rank) {
  __shared__ unsigned long long s_mask[kWaves][kMaxExperts];
  __shared__ int s_base[kWaves][kMaxExperts];
  const int wv = wave_id(), lane = lane_id();
  for (int i = threadIdx.x; i < kWaves * kMaxExperts; i += kThreads) (&s_mask[0][0])[i] = 0ull;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kDispatchTokensPerBlock + threadIdx.x;
  const bool valid = t < T;
  if (valid) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if ((unsigned)e < (unsigned)E) atomicOr(&s_mask[wv][e], 1ull << lane);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) {
    int run = 0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
      s_base[q][e] = run;
      run += __popcll(s_mask[q][e]);
    }
    blk_counts[(int64_t)blockIdx.x * E + e] = run;
  }
  __syncthreads();
  if (valid) {
    const unsigned long long lower = (1ull << lane) - 1ull;
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      int r = -1;
      if ((unsigned)e < (unsigned)E) r = s_base[wv][e] + __popcll(s_mask[wv][e] & lower);
      local_rank[t * k + j] = r;
    }
  }
}

__global__ __launch_bounds__(kMaxExperts) void dispatch_scan_kernel(
    int64_t nblk, int E, int64_t capacity, int32_t* __restrict__ blk_counts,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ zero,
    int nzero) {
  __shared__ int s_kept[kMaxExperts];
  const int e = threadIdx.x;
  if (zero)  // a later kernel's counters (see launch_dispatch)
    for (int i = e; i < nzero; i += blockDim.x) zero[i] = 0;
  if (e < E) {
    int run = 0;
    constexpr int kChunk = 16;  // independent loads in flight
    for (int64_t b0 = 0; b0 < nblk; b0 += kChunk) {
      int c[kChunk];
#pragma unroll
      for (int q = 0; q < kChunk; ++q) c[q] = (b0 + q < nblk) ? blk_counts[(b0 + q) * E + e] : 0;
#pragma unroll
      for (int q = 0; q < kChunk; ++q) {
        if (b0 + q < nblk) blk_counts[(b0 + q) * E + e] = run;  // becomes the block's base
        run += c[q];
      }
    }
    if (counts) counts[e] = run;
    s_kept[e] = (capacity < 0) ? run : (int)min((int64_t)run, capacity);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int q = 0; q < E; ++q) {
      offsets[q] = acc;
      acc += s_kept[q];
    }
    offsets[E] = acc;
  }
}

template <typename U>  // copy unit (uint4, uint32_t or uint16_t)
__global__ __launch_bounds__(kThreads) void dispatch_place_kernel(
    int64_t T, int k, int E, int64_t capacity, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ local_rank,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ slot_row,
    const U* __restrict__ x, U* __restrict__ x_perm, int64_t row_units, bool padded) {
  const int lane = lane_id();
  const int64_t t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWaves + wave_id()));
  if (t >= T) return;
  const int64_t b = t / kDispatchTokensPerBlock;
  for (int j0 = 0; j0 < k; j0 += kWave) {
    const int j = j0 + lane;
    int row = -1;
    if (j < k) {
      const int64_t s = t * k + j;
      const int e = idx[s];
      const int lr = local_rank[s];
      if ((unsigned)e < (unsigned)E && lr >= 0) {
        const int r = blk_base[b * E + e] + lr;
        if (capacity < 0 || r < capacity) {
          row = padded ? (int)((int64_t)e * capacity + r) : offsets[e] + r;
          perm[row] = (int32_t)s;
        }
      }
      slot_row[s] = row;
    }
    if (x_perm) {
      const int nj = min(kWave, k - j0);
      const U* src = x + t * row_units;
      for (int64_t c = lane; c < row_units; c += kWave) {
        const U v = src[c];
        for (int jj = 0; jj < nj; ++jj) {
          const int rr = __shfl(row, jj);
          if (rr >= 0) x_perm[(int64_t)rr * row_units + c] = v;
        }
      }
    }
  }
}

// Empty rows of the padded batches, one wave per row: row i of batch e is empty when i is not
// below kept_e = offsets[e + 1] - offsets[e] (the compact offsets of the scan): perm = -1 and,
// with a copy, a zero row. Block 0 also writes the batch starts e * capacity and, without a
// copy, clears `zero_row` (one row of x: the GEMM reads it for the empty rows).
template <typename U>
__global__ __launch_bounds__(kThreads) void dispatch_pad_fill_kernel(
    int E, int64_t capacity, const int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    U* __restrict__ x_pad, int64_t row_units, int32_t* __restrict__ pad_offsets,
    U* __restrict__ zero_row) {
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i <= E; i += kThreads)
      pad_offsets[i] = (int32_t)((int64_t)i * capacity);
    if (zero_row) {
      U zero;
      __builtin_memset(&zero, 0, sizeof(U));
      for (int64_t c = threadIdx.x; c < row_units; c += kThreads) zero_row[c] = zero;
    }
  }
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave_id();
  if (row >= (int64_t)E * capacity) return;
  const int e = (int)(row / capacity);
  const int64_t i = row - (int64_t)e * capacity;
  if (i < offsets[e + 1] - offsets[e]) return;  // a kept slot's row
  if (lane_id() == 0) perm[row] = -1;
  if (x_pad) {
    U zero;
    __builtin_memset(&zero, 0, sizeof(U));
    for (int64_t c = lane_id(); c < row_units; c += kWave) x_pad[row * row_units + c] = zero;
  }
}

}  // namespace

int64_t dispatch_blocks(const Problem& p) {
  return (p.T + kDispatchTokensPerBlock - 1) / kDispatchTokensPerBlock;
}

hipError_t launch_dispatch(const Problem& p, const int32_t* idx, const void* x, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* slot_row, void* x_perm,
                           int32_t* blk_counts, int32_t* local_rank, hipStream_t s,
                           int32_t* zero, int nzero, int32_t* pad_offsets, void* zero_row) {
  const bool padded = pad_offsets != nullptr;
  const int64_t nblk = dispatch_blocks(p);
  if (nblk > 0) {
    hipLaunchKernelGGL(dispatch_rank_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, s, p.T,
                       p.top_k, p.E, idx, blk_counts, local_rank);
  }
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kMaxExperts), 0, s, nblk, p.E,
                     p.capacity, blk_counts, counts, offsets, zero, nzero);
  const int64_t es = (p.dtype == MOE_BF16) ? 2 : 4;
  const int64_t row_bytes = p.D * es;
  const bool al16 = ((uintptr_t)x % 16 == 0) && ((uintptr_t)x_perm % 16 == 0);
  const int unit = (x_perm && row_bytes % 16 == 0 && al16) ? 16
                   : (x_perm && row_bytes % 4 == 0)        ? 4
                                                           : 2;
  if (p.T > 0) {
    const unsigned grid = (unsigned)((p.T + kWaves - 1) / kWaves);
    if (unit == 16)
      hipLaunchKernelGGL(dispatch_place_kernel<uint4>, dim3(grid), dim3(kThreads), 0, s, p.T,
                         p.top_k, p.E, p.capacity, idx, blk_counts, local_rank, offsets, perm,
                         slot_row, (const uint4*)x, (uint4*)x_perm, row_bytes / 16, padded);
    else if (unit == 4)
      hipLaunchKernelGGL(dispatch_place_kernel<uint32_t>, dim3(grid), dim3(kThreads), 0, s, p.T,
                         p.top_k, p.E, p.capacity, idx, blk_counts, local_rank, offsets, perm,
                         slot_row, (const uint32_t*)x, (uint32_t*)x_perm, row_bytes / 4, padded);
    else
      hipLaunchKernelGGL(dispatch_place_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, s, p.T,
                         p.top_k, p.E, p.capacity, idx, blk_counts, local_rank, offsets, perm,
                         slot_row, (const uint16_t*)x, (uint16_t*)x_perm, row_bytes / 2, padded);
  }
  if (padded) {
    const int64_t rows = (int64_t)p.E * p.capacity;
    const unsigned grid = (unsigned)std::max<int64_t>(1, (rows + kWaves - 1) / kWaves);
    if (unit == 16)
      hipLaunchKernelGGL(dispatch_pad_fill_kernel<uint4>, dim3(grid), dim3(kThreads), 0, s, p.E,
                         p.capacity, offsets, perm, (uint4*)x_perm, row_bytes / 16, pad_offsets,
                         (uint4*)zero_row);
    else if (unit == 4)
      hipLaunchKernelGGL(dispatch_pad_fill_kernel<uint32_t>, dim3(grid), dim3(kThreads), 0, s,
                         p.E, p.capacity, offsets, perm, (uint32_t*)x_perm, row_bytes / 4,
                         pad_offsets, (uint32_t*)zero_row);
    else
      hipLaunchKernelGGL(dispatch_pad_fill_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, s,
                         p.E, p.capacity, offsets, perm, (uint16_t*)x_perm, row_bytes / 2,
                         pad_offsets, (uint16_t*)zero_row);
  }
  return hipGetLastError();
}

}  // namespace moe

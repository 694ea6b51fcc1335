// Shared device helpers and the internal launcher interface of the MoE library.
// Written for gfx950 (CDNA4): 64-lane wavefronts, bf16 MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 256;

// Tokens per block of the routing kernel; the per-block partial sums of the
// router probabilities and the per-block expert counts are indexed by it.
constexpr int kRouteTokensPerBlock = 16;
// Tokens per block of the dispatch count/rank kernel (4 waves, one token per lane).
constexpr int kDispatchTokensPerBlock = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// float -> bfloat16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ double load_as_f64(const float* p, int64_t i) { return (double)p[i]; }
__device__ __forceinline__ double load_as_f64(const uint16_t* p, int64_t i) {
  return (double)bf16_to_f32(p[i]);
}
__device__ __forceinline__ float load_as_f32(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_as_f32(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}
__device__ __forceinline__ void store_from_f32(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_from_f32(uint16_t* p, int64_t i, float v) {
  p[i] = f32_to_bf16(v);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// ---------------------------------------------------------------------------------------
// Internal launchers (one translation unit each). All return hipGetLastError().

struct Problem {
  int64_t T, D, DH, D_out;
  int E, top_k;
  int64_t capacity;  // -1: no limit
  int dtype, kind;
  int64_t slots() const { return T * (int64_t)top_k; }
};

// Routing: logits, softmax, top-k, gates, per-block probability sums and counts.
// `ws` is the routing scratch (route_ws_bytes bytes, 256-byte aligned).
int64_t route_blocks(const Problem& p);
int route_splits(const Problem& p);
size_t route_ws_bytes(const Problem& p);
// Router options: noise (w_noise (D, E) in the layer's dtype and the (T, E) float32 draw, or
// both null) and renormalisation of the gates.
struct RouteOpts {
  const void* w_noise = nullptr;
  const float* noise = nullptr;
  bool renorm = true;
};
// `uncertified` (nullable, device) receives the number of tokens whose logits were
// recomputed in float64 (always 0 for float32 layers, which are float64 throughout).
hipError_t launch_route(const Problem& p, const void* x, const void* w_router, const float* bias,
                        const RouteOpts& o, int32_t* idx, float* gates, float* logits_out,
                        int32_t* uncertified, void* ws, hipStream_t s);
// Sum of the per-block partials -> aux loss (and the per-expert counts, if asked). With
// `importance` (nullable) also the importance loss from the final idx / gates.
hipError_t launch_aux_finalize(const Problem& p, void* ws, float* aux, int32_t* counts_out,
                               hipStream_t s, const int32_t* idx = nullptr,
                               const float* gates = nullptr, float* importance = nullptr);

// Routing with its losses in one call: the fused bf16 path (prep + one routing kernel + one
// block that forms the loss and the counts) when it applies, else launch_route +
// launch_aux_finalize. With `dispatch_done` (nullable) and `offsets_out`, the fused path
// instead leaves the loss, the counts, the offsets and the placement to
// launch_place_after_route, which the caller must then run with the same aux / counts /
// uncertified pointers (it writes perm and slot_row as launch_dispatch does); *dispatch_done
// tells which happened.
hipError_t launch_route_full(const Problem& p, const void* x, const void* w_router,
                             const float* bias, const RouteOpts& o, int32_t* idx, float* gates,
                             float* logits_out, int32_t* uncertified, float* aux,
                             int32_t* counts_out, float* importance, void* ws, hipStream_t s,
                             int32_t* offsets_out = nullptr, bool* dispatch_done = nullptr);
hipError_t launch_place_after_route(const Problem& p, const int32_t* idx, void* ws, float* aux,
                                    int32_t* counts_out, int32_t* uncertified,
                                    int32_t* offsets, int32_t* perm, int32_t* slot_row,
                                    hipStream_t s, int32_t* zero = nullptr, int nzero = 0,
                                    float* importance = nullptr);
// route_fused.hip (used through the two calls above)
bool fused_route_applies(const Problem& p, const RouteOpts& o, bool importance);
size_t fused_route_ws_bytes(const Problem& p);
hipError_t launch_route_fused(const Problem& p, const void* x, const void* w_router,
                              const float* bias, bool renorm, int32_t* idx, float* gates,
                              float* logits_out, void* fws, hipStream_t s,
                              bool importance = false, const void* w_noise = nullptr,
                              const float* noise = nullptr);
// perm null: one block forms the loss and the counts (and the offsets, if given) only
hipError_t launch_place_fused(const Problem& p, const int32_t* idx, const void* fws, float* aux,
                              int32_t* counts_out, int32_t* uncertified, int32_t* offsets,
                              int32_t* perm, int32_t* slot_row, hipStream_t s, int32_t* zero,
                              int nzero, float* importance = nullptr);

// Dispatch: per-block histogram + stable local ranks, scan + capacity, placement (+ copy).
int64_t dispatch_blocks(const Problem& p);
// `zero` (nullable): nzero int32 that the scan kernel sets to 0 on the way (the GEMMs'
// K-split tickets and work queue of the same call, which saves a launch).
// `pad_offsets` (nullable; needs a capacity): the capacity-padded layout. perm (E * capacity)
// and slot_row then index padded rows e * capacity + rank, empty rows get perm -1 and a zero
// row in x_perm, `offsets` still receives the compact offsets (kept rows) and pad_offsets
// (E + 1) the batch starts e * capacity.
hipError_t launch_dispatch(const Problem& p, const int32_t* idx, const void* x,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_row,
                           void* x_perm, int32_t* blk_counts, int32_t* local_rank,
                           hipStream_t s, int32_t* zero = nullptr, int nzero = 0,
                           int32_t* pad_offsets = nullptr, void* zero_row = nullptr);

// Backward of the layer (backward.hip): workspace bytes and the launch sequence.
// A training forward's saved state (byte offsets in the caller's buffer, 256-byte aligned):
// the float32 logits (T, E), the permutation (T*k), and per expert row (T*k rows, p's dtype)
// the pre-activations a (ReLU, SwiGLU) and b (SwiGLU), the hidden h and the expert outputs y.
struct SavedLayout {
  size_t logits, perm, a, b, h, y, total;
};
SavedLayout saved_layout(const Problem& q);
// The experts' forward on the kept rows (row r reads token row perm[r] / top_k of x), keeping
// a, b, h and y; the same kernels serve the training forward and the backward's recompute.
hipError_t run_experts_saving(const Problem& q, const void* x, const int32_t* perm,
                              const int32_t* offsets, const void* w1, const void* w3,
                              const void* w2, void* a, void* b, void* h, void* y,
                              float* split_ws, int64_t split_slots, int32_t* split_ctr,
                              int32_t* queue, int ncu, hipStream_t s);
hipError_t launch_backward_saved(const Problem& q, const int32_t* idx, const float* gates,
                                 const int32_t* counts, const int32_t* offsets,
                                 const int32_t* slot_row, const void* saved, const void* x,
                                 const void* w_router, const void* w1, const void* w3,
                                 const void* w2, const void* dout, float d_aux, void* dx,
                                 float* dw_router, float* dbias, void* dw1, void* dw3, void* dw2,
                                 void* ws, hipStream_t s);
size_t backward_ws_bytes(const Problem& q);
hipError_t launch_backward(const Problem& q, const void* x, const void* w_router, const float* bias,
                           const void* w1, const void* w3, const void* w2, const void* dout,
                           float d_aux, void* dx, float* dw_router, float* dbias, void* dw1,
                           void* dw3, void* dw2, void* ws, hipStream_t s);

// Grouped expert GEMM over expert-ordered rows.
enum Epilogue { EPI_NONE = 0, EPI_RELU = 1, EPI_SWIGLU = 2 };
struct GroupedGemm {
  const void* A;            // rows of length K (row-major), element type = dtype
  int64_t lda;
  const int32_t* a_gather;  // optional: row r of A is A[a_gather[r] / gather_div]
  int gather_div;
  // optional (bf16 256 x 256 kernel only): rows whose a_gather entry is negative read this
  // row of lda zeros instead (the empty rows of capacity-padded batches)
  const void* a_zero;
  const void* B0;           // (E, K, N) row-major
  const void* B1;           // second (E, K, N) for SwiGLU, else null
  void* C;                  // (rows, N) row-major, ldc = N
  const int32_t* offsets;   // (E+1) expert row offsets, device
  int E;
  int64_t K, N;
  int64_t max_rows;         // upper bound of offsets[E] (grid sizing)
  int epilogue;
  int dtype;
  // K-split tail (bf16 256x256 kernel only; null split_ws: no split). split_ws holds
  // split_slots (at most kSplitSlots) partial tiles of kSplitSlotFloats floats, split_ctr
  // kSplitSlots tickets; a launch that could need more slots does not split. ncu = compute
  // units used to size waves (at most kSplitSlots, a multiple of 8).
  float* split_ws;
  int64_t split_slots;
  int32_t* split_ctr;
  int ncu;
  // Work queue of the 256 x 256 kernel (kQueueInts int32, zero on entry, left zero): one
  // counter per XCD and a count of finished blocks. Null: the 256 x 256 kernel is not used.
  int32_t* queue;
  // Optional (null: none): events that bracket the GEMM kernel itself (recorded by its
  // dispatch where the kernel supports that, else recorded on the stream around it).
  hipEvent_t ev_start, ev_stop;
  // B0 stored K-major, (E, N, K) row-major (a forward weight used transposed, for the
  // backward's dgrad). Only with EPI_NONE and the 256 x 256 kernel (bf16, K % 128 == 0).
  bool b_kmajor;
  // K-grouped (the backward's wgrad, C_g = A_g^T B_g for each group g): group g owns output
  // rows offsets[g] .. offsets[g + 1] (offsets[g] = g * M, M = group_rows), and its K range is
  // k_offsets[g] .. k_offsets[g + 1] (multiples of 128, at least 128 wide). A holds the groups'
  // transposed operands side by side, (M, lda) row-major: row m of group g starts at column
  // k_offsets[g]. B's K-row i of group g is row b_offsets[g] + i of B0 ((rows, N) row-major);
  // every K-row read must be in bounds and finite, and the A columns past a group's own
  // K-rows zero. Only with EPI_NONE, no split, and the 256 x 256 kernel.
  bool k_grouped;
  const int32_t* k_offsets;
  const int32_t* b_offsets;
  int64_t group_rows;
  // Optional (null: not stored; 256 x 256 kernel only): the pre-activations of an EPI_RELU or
  // EPI_SWIGLU product, in C's layout and type: pre_a = A B0 (before the ReLU, or the SwiGLU
  // gate input), pre_b = A B1 (SwiGLU only).
  void* pre_a;
  void* pre_b;
};
constexpr int kSplitSlots = 256;
constexpr int kQueueInts = 16;
constexpr int64_t kSplitSlotFloats = 256 * 256;
// Compute units of the current device, capped at kSplitSlots (0 when not a multiple of 8).
int device_split_cus();
// Partial-tile slots that a K split of a bf16 product (max_rows rows over E experts, K x N,
// SwiGLU column tiles or not) can use: 0 when K is too short to split.
int64_t gemm_bf16_split_slots(int64_t max_rows, int E, int64_t K, int64_t N, bool swiglu);
hipError_t launch_grouped_gemm(const GroupedGemm& g, hipStream_t s);
// bf16, 256 x 256 tiles (expert_gemm_bf16.hip). The K-split tickets (split_ctr) must be zero
// on entry; the kernel leaves them zero.
hipError_t launch_grouped_gemm_bf16_256(const GroupedGemm& g, hipStream_t s);
hipError_t launch_zero_tickets(int32_t* tickets, int n, hipStream_t s);

// Combine: out[t] = sum_j gates[t,j] * y[slot_row[t*k+j]].
hipError_t launch_combine(const Problem& p, const void* y, const int32_t* slot_row,
                          const float* gates, void* out, hipStream_t s);

}  // namespace moe

/*
 * moe.h -- C ABI of the MI355X (gfx950) top-k Mixture-of-Experts layer forward.
 *
 * The layer, as the source pages define it:
 *   logits = x @ W_router (+ bias)                      (T, E)
 *   probs  = softmax(logits) per row
 *   expert_indices[t] = the top_k experts by descending logit (ties: lower index)
 *   gates[t]          = softmax of those top_k logits
 *   aux_loss = E * sum_e f_e * P_e,  f_e = count_e / (T * top_k),  P_e = mean_t probs[t, e]
 *   capacity = floor(capacity_factor * T * top_k / E) slots per expert (when > 0); an
 *              expert keeps its routed tokens in ascending token order up to capacity and
 *              drops the rest
 *   output[t] = sum over kept slots j of gates[t, j] * expert_{expert_indices[t, j]}(x[t])
 * Sources: ML Grind "Mixture-of-Experts (MoE) Routing" (Algorithm; Inputs; Expected Return
 * Format; Edge cases and conventions; Follow-up) and "Mixture of Experts: the Sparsely-Gated
 * Layer" (The one formula; Switch: top-1, one loss, and a rate limit; The code).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is a DEVICE pointer unless marked "host". The library never
 *   allocates or frees memory and keeps no state between calls; the caller owns every
 *   buffer. Scratch memory comes from the caller's workspace `ws` of `ws_bytes` bytes
 *   (256-byte aligned), sized by moe_workspace_size().
 * - Matrices are row-major. Weights follow the pages' "x @ W" convention, (in, out):
 *   W_router (D, E); w1, w3 (E, D, DH); w2 (E, DH, D_out); a linear expert is w1 (E, D, D_out).
 * - `dtype` is the storage type of x, the router and expert weights, x_perm, y_perm and out.
 *   MOE_F32: float32 storage, float32 expert arithmetic. MOE_BF16: bfloat16 storage, float32
 *   accumulation, the expert hidden activation rounded to bfloat16 (round to nearest even).
 *   Routing decisions (top-k), gates and the loss are computed from logits that equal the
 *   exact logits to within a certified bound; a token whose decision that bound cannot
 *   certify is recomputed in float64. Gates and aux_loss are float32, indices int32.
 * - A "slot" is a (token t, rank j) pair with id s = t * top_k + j. Buffers indexed by rows
 *   of expert-ordered data are sized for the worst case, T * top_k rows; the number of kept
 *   rows R = expert_offsets[E] stays on the device (the host never synchronises).
 * - Arguments are checked on the host before anything is launched. On any error nothing is
 *   written and nothing is launched. After the launches, a launch failure is reported as
 *   MOE_ERR_HIP; faults during execution surface at the caller's next stream
 *   synchronisation. NaN or Inf inputs give unspecified (but memory-safe) results.
 * - All work is enqueued on `stream` (0 = the null stream), in stream order; calls are
 *   reentrant. Outputs must not alias inputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a null required pointer, a size out of range, top_k not in [1, E] */
  MOE_ERR_UNSUPPORTED = 2, /* E > 256, an unknown dtype/kind, widths not multiples of 8 in bf16 */
  MOE_ERR_WORKSPACE = 3,   /* ws_bytes smaller than moe_workspace_size(), or ws misaligned */
  MOE_ERR_HIP = 4,         /* a HIP launch error */
  MOE_ERR_SCRATCH_LIMIT = 5 /* moe_route_noalloc: the problem needs more routing scratch than
                               MOE_NOALLOC_SCRATCH_BYTES */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* The expert FFN (names as on the pages: D, DH, NEXP, TOPK).
 * LINEAR: x @ W (ML Grind, Background).
 * RELU2:  relu(x @ Wh) @ Wo, no biases (Sparsely-Gated Layer, expert_forward).
 * SWIGLU: (silu(x @ W1) * (x @ W3)) @ W2, silu(z) = z / (1 + exp(-z)). */
typedef enum moe_expert_kind {
  MOE_EXPERT_LINEAR = 0,
  MOE_EXPERT_RELU2 = 1,
  MOE_EXPERT_SWIGLU = 2
} moe_expert_kind;

/* The problem statement (host struct). */
typedef struct moe_problem {
  int64_t T;              /* tokens, >= 0 (T = 0 is a valid empty call) */
  int64_t D;              /* model width d, >= 1 */
  int64_t DH;             /* expert hidden width, >= 1 (ignored for LINEAR) */
  int64_t D_out;          /* expert output width, >= 1 */
  int32_t E;              /* experts, 1..256 */
  int32_t top_k;          /* experts per token, 1..E */
  double capacity_factor; /* <= 0: no capacity limit */
  int32_t dtype;          /* moe_dtype */
  int32_t kind;           /* moe_expert_kind */
} moe_problem;

/* Human-readable name of a status code (static storage, never NULL). Takes any int: a value
 * that is not a moe_status gives "unknown moe_status". */
const char* moe_status_string(int status);

/* Checks a problem statement (host only). Returns MOE_OK, MOE_ERR_INVALID_ARG or
 * MOE_ERR_UNSUPPORTED. */
moe_status moe_check_problem(const moe_problem* p);

/* Slots per expert: floor(capacity_factor * T * top_k / E) computed in double, or -1 when
 * capacity_factor <= 0 (no limit). Host only; -2 for an invalid problem.
 * (Sparsely-Gated Layer, "Switch: top-1, one loss, and a rate limit".) */
int64_t moe_capacity(const moe_problem* p);

/* Bytes of workspace that moe_forward needs; every other entry point needs at most this
 * much. Host only; 0 for an invalid problem. */
size_t moe_workspace_size(const moe_problem* p);

/* Router, softmax, top-k, gates and the Switch loss (ML Grind, Algorithm steps 1, 2 and the
 * load-balancing step).
 *   x (T, D), w_router (D, E) in p->dtype; router_bias (E) float32 or NULL.
 *   Outputs: expert_indices (T, top_k) int32, best first; gates (T, top_k) float32, each row
 *   summing to 1; aux_loss (1) float32; expert_counts (E) int32 routed slots per expert before
 *   capacity, or NULL; logits_out (T, E) float32 copy of the router logits, or NULL;
 *   uncertified (1) int32, or NULL: the number of tokens whose top-k order the fast bf16
 *   logits could not certify and that were therefore recomputed in float64. 0 wherever every
 *   logit is already exact to float64 rounding: MOE_F32, and MOE_BF16 with 8 <= E <= 64,
 *   E % 8 == 0, D % 64 == 0 (float64 matrix-core sums of the exact products of the bf16
 *   inputs); with router noise (moe_route_ex) where also E <= 32, the noise router's E columns
 *   then summed beside the logits' in the same pass.
 *   With T = 0, aux_loss is 0 and expert_counts are zeros. */
moe_status moe_route(const moe_problem* p, const void* x, const void* w_router,
                     const float* router_bias, int32_t* expert_indices, float* gates,
                     float* aux_loss, int32_t* expert_counts, float* logits_out,
                     int32_t* uncertified, void* ws, size_t ws_bytes, hipStream_t stream);

/* Size of the fixed device array that moe_route_noalloc uses as its scratch (32 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)

/* moe_route without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, outputs and errors as moe_route (no router options), minus ws and ws_bytes; the
 * results are bit-identical to moe_route's for the same inputs.
 *   Scratch: a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one per
 *   device, held from the library's load until the process ends. Its device address is looked
 *   up once per device, on that device's first call. The call allocates nothing (no hipMalloc,
 *   hipFree or allocating library routine) and clears what must start at zero itself.
 *   Every call on a device shares that device's array, so calls that overlap on one device
 *   (concurrent streams or host threads) race and give undefined results; calls on one stream
 *   are safe. `stream` must belong to the current device (else MOE_ERR_INVALID_ARG).
 *   MOE_ERR_SCRATCH_LIMIT (nothing written or launched) when the routing scratch this problem
 *   needs exceeds the array; it grows with T and E (the five workloads of the pages' shapes
 *   need at most about 19 MiB). */
moe_status moe_route_noalloc(const moe_problem* p, const void* x, const void* w_router,
                             const float* router_bias, int32_t* expert_indices, float* gates,
                             float* aux_loss, int32_t* expert_counts, float* logits_out,
                             int32_t* uncertified, hipStream_t stream);

/* Dispatch (ML Grind, Algorithm step 3: each expert's tokens collected; capacity as in the
 * Sparsely-Gated Layer page's moe_forward, earlier tokens kept before later ones).
 *   expert_indices (T, top_k) int32 in [0, E) with distinct entries per row (unchecked);
 *   x (T, D) in p->dtype, or NULL when x_perm is NULL.
 *   Outputs: expert_counts (E) int32 before capacity; expert_offsets (E+1) int32, the
 *   exclusive prefix sum of kept_e = min(count_e, capacity); perm (T*top_k) int32, perm[r] =
 *   the slot placed at expert-ordered row r for r < R (rows of one expert in ascending token
 *   order; entries from R on are left untouched); slot_row (T*top_k) int32, the row of slot s
 *   or -1 when s was dropped; x_perm (T*top_k, D) in p->dtype, x_perm[r] = x[perm[r] / top_k]
 *   for r < R, or NULL to skip the copy. */
moe_status moe_dispatch(const moe_problem* p, const int32_t* expert_indices, const void* x,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                        int32_t* slot_row, void* x_perm, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* The experts, each on its own rows only (ML Grind, Algorithm step 3 and Constraints):
 * y_perm[r] = expert_e(x_perm[r]) for expert_offsets[e] <= r < expert_offsets[e+1].
 *   x_perm (T*top_k, D); w1 (E, D, DH) or (E, D, D_out) for LINEAR; w3 (E, D, DH) for SWIGLU,
 *   else NULL; w2 (E, DH, D_out), NULL for LINEAR; y_perm (T*top_k, D_out); all in p->dtype.
 *   Rows from R on are neither read nor written. */
moe_status moe_expert_ffn(const moe_problem* p, const void* x_perm, const int32_t* expert_offsets,
                          const void* w1, const void* w3, const void* w2, void* y_perm, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* Gate-weighted combine back in token order (ML Grind, Algorithm step 3 formula):
 * out[t] = sum_{j < top_k, slot_row[t*top_k+j] >= 0} gates[t, j] * y_perm[slot_row[...]],
 * accumulated in float32 in ascending j and rounded once to p->dtype. A dropped slot adds
 * nothing and gates are not renormalised; a token with every slot dropped gets zeros.
 *   y_perm (T*top_k, D_out); slot_row (T*top_k) int32; gates (T, top_k) float32;
 *   out (T, D_out). No workspace. */
moe_status moe_combine(const moe_problem* p, const void* y_perm, const int32_t* slot_row,
                       const float* gates, void* out, hipStream_t stream);

/* The whole layer: route, dispatch, experts, combine, loss, on one stream, with no host
 * synchronisation. Arguments as in the stage functions above; expert_counts,
 * expert_offsets and slot_row are outputs (required). */
moe_status moe_forward(const moe_problem* p, const void* x, const void* w_router,
                       const float* router_bias, const void* w1, const void* w3, const void* w2,
                       void* out, int32_t* expert_indices, float* gates, float* aux_loss,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* slot_row,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Stages of moe_forward, in launch order, for moe_forward_timed. */
enum {
  MOE_STAGE_ROUTE = 0,       /* router GEMM, softmax, top-k, gates; loss partials and loss */
  MOE_STAGE_DISPATCH = 1,    /* histogram + ranks, scan + capacity, placement */
  MOE_STAGE_EXPERT_UP = 2,   /* first expert GEMM (+ activation); the whole expert if LINEAR */
  MOE_STAGE_EXPERT_DOWN = 3, /* second expert GEMM (empty for LINEAR) */
  MOE_STAGE_COMBINE = 4,     /* gate-weighted combine */
  MOE_NUM_STAGES = 5
};

/* moe_forward with per-stage timing: `stage_events` holds 2 * MOE_NUM_STAGES events that the
 * caller created (hipEventCreate), or NULL entries for stages not to be timed. For the two
 * expert stages the pair brackets the GEMM kernel itself (recorded by the kernel's dispatch,
 * which adds nothing to the stream); for the other stages event 2s is recorded on `stream`
 * right before stage s and event 2s+1 right after it (each such record can leave the device
 * idle for a few microseconds). hipEventElapsedTime(events[2s], events[2s+1]) is then the
 * device time of stage s. NULL stage_events behaves as moe_forward.
 * (Per-stage device timing of the layer; the work is identical to moe_forward.) */
moe_status moe_forward_timed(const moe_problem* p, const void* x, const void* w_router,
                             const float* router_bias, const void* w1, const void* w3,
                             const void* w2, void* out, int32_t* expert_indices, float* gates,
                             float* aux_loss, int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* slot_row, void* ws, size_t ws_bytes, hipStream_t stream,
                             hipEvent_t* stage_events);

/* ---- Router options and the capacity-padded layout --------------------------------------
 * Options of the router on the page "Mixture of Experts: the Sparsely-Gated Layer" and of the
 * Switch layer's fixed-size expert batches (host struct; NULL or all zero = the layer above:
 * no noise, renormalised gates, compact expert rows, no importance loss).
 *   w_noise, noise: router noise ("The one formula", the + noise row; router() stage (2) in
 *     "The code"). w_noise (D, E) in p->dtype; noise (T, E) float32, the standard-normal draw,
 *     supplied by the caller (the library draws nothing, so every call is deterministic). The
 *     decision logits become logits + noise[t, e] * softplus(x_t . w_noise[:, e]), and the
 *     probabilities, top-k, gates and both losses use them. Both NULL or both set.
 *   no_renormalise: nonzero = the gates are the chosen experts' probabilities over all E
 *     experts (router(..., renormalise=False): stage (5) skipped), so a gate row sums to at
 *     most 1. These gates need all E logits to the gates' accuracy: where the logits are not
 *     exact already (see moe_route), every token's are recomputed in float64 and
 *     `uncertified` counts every token.
 *   padded: nonzero = expert batches padded to the capacity ("Switch: top-1, one loss, and a
 *     rate limit": experts run as fixed-size batches); needs capacity_factor > 0. Expert e's
 *     kept slots take rows e * capacity + rank (rank in token order) and the rest of its batch
 *     is zero rows, which the expert GEMMs compute anyway (the padding cost the page names).
 *   importance_loss: device float32 (1), or NULL: Shazeer's importance loss ("Hot shards: the
 *     load-balancing loss", importance_loss()), the squared coefficient of variation
 *     (population standard deviation over the mean) of the per-expert sums of the gates;
 *     0 when T = 0. Deterministic (fixed-order sums). */
typedef struct moe_options {
  const void* w_noise;
  const float* noise;
  int32_t no_renormalise;
  int32_t padded;
  float* importance_loss;
} moe_options;

/* Bytes of workspace that the *_ex entry points need with these options (opts may be NULL;
 * then equal to moe_workspace_size). Host only; 0 for an invalid problem or options
 * (padded without a capacity). */
size_t moe_workspace_size_ex(const moe_problem* p, const moe_options* opts);

/* moe_route with options (opts->padded plays no part here). Errors as moe_route, plus
 * MOE_ERR_INVALID_ARG when exactly one of w_noise and noise is set. */
moe_status moe_route_ex(const moe_problem* p, const moe_options* opts, const void* x,
                        const void* w_router, const float* router_bias, int32_t* expert_indices,
                        float* gates, float* aux_loss, int32_t* expert_counts,
                        float* logits_out, int32_t* uncertified, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Dispatch into the capacity-padded layout (Sparsely-Gated Layer page, "Switch: top-1, one
 * loss, and a rate limit"; earlier tokens kept first, as in moe_dispatch). Needs
 * capacity_factor > 0 (else MOE_ERR_INVALID_ARG); with capacity 0 every slot is dropped.
 *   expert_indices, x as in moe_dispatch. Outputs: expert_counts (E) int32 before capacity;
 *   expert_offsets (E+1) int32, the batch starts e * capacity (what moe_expert_ffn_ex takes);
 *   perm (E * capacity) int32, the slot of each padded row or -1 for an empty row; slot_row
 *   (T*top_k) int32, the padded row of each slot or -1 when dropped; x_pad (E * capacity, D)
 *   in p->dtype, each kept slot's token row and zero rows elsewhere, or NULL to skip the copy.
 *   Workspace: moe_workspace_size_ex with padded set. */
moe_status moe_dispatch_padded(const moe_problem* p, const int32_t* expert_indices,
                               const void* x, int32_t* expert_counts, int32_t* expert_offsets,
                               int32_t* perm, int32_t* slot_row, void* x_pad, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* moe_expert_ffn over a padded layout: as moe_expert_ffn, except that expert_offsets[E] may
 * be up to max(T * top_k, E * capacity) rows (x_perm and y_perm sized for that many) when
 * opts->padded; the workspace is moe_workspace_size_ex's. */
moe_status moe_expert_ffn_ex(const moe_problem* p, const moe_options* opts, const void* x_perm,
                             const int32_t* expert_offsets, const void* w1, const void* w3,
                             const void* w2, void* y_perm, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* moe_forward_timed with options (stage_events may be NULL). With opts->padded,
 * expert_offsets receives the batch starts e * capacity and slot_row the padded rows, as in
 * moe_dispatch_padded, and the dispatch stage includes the padded copy of x. */
moe_status moe_forward_ex(const moe_problem* p, const moe_options* opts, const void* x,
                          const void* w_router, const float* router_bias, const void* w1,
                          const void* w3, const void* w2, void* out, int32_t* expert_indices,
                          float* gates, float* aux_loss, int32_t* expert_counts,
                          int32_t* expert_offsets, int32_t* slot_row, void* ws, size_t ws_bytes,
                          hipStream_t stream, hipEvent_t* stage_events);

/* ---- Backward -------------------------------------------------------------------------------
 * Gradients of L = sum(out * dout) + d_aux * aux_loss for the layer of moe_forward (no router
 * noise, renormalised gates), by the chain rule through its steps in reverse. The routing
 * decisions and the drop set are piecewise constant, so the gradient flows through the gates
 * and through P in the Switch loss; f, a count, is a step function of the logits and has none
 * (ML Grind page, the load-balancing step; Sparsely-Gated Layer page, Hot shards). relu'(0)
 * is taken as 0; silu'(z) = s (1 + z (1 - s)) with s = sigmoid(z).
 *   Inputs: x, w_router, router_bias (nullable), w1, w3, w2 as in moe_forward; dout (T, D_out)
 *   in p->dtype; d_aux (host) the weight of the Switch loss in L.
 *   Outputs (overwritten): dx (T, D) and dw1, dw3 (SwiGLU only, else NULL), dw2 (not LINEAR,
 *   else NULL) in p->dtype with the weights' shapes; dw_router (D, E) float32; dbias (E)
 *   float32 or NULL. An expert that kept no token gets a zero gradient.
 *   The call recomputes the forward quantities it needs (routing, dispatch, the experts'
 *   pre-activations and outputs) with the forward's kernels; it needs no saved state.
 *   Workspace: moe_backward_workspace_size bytes. With T = 0 nothing is written. */
size_t moe_backward_workspace_size(const moe_problem* p);

moe_status moe_backward(const moe_problem* p, const void* x, const void* w_router,
                        const float* router_bias, const void* w1, const void* w3, const void* w2,
                        const void* dout, float d_aux, void* dx, float* dw_router, float* dbias,
                        void* dw1, void* dw3, void* dw2, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* ---- Training forward and the backward from its saved state ------------------------------
 * The backward above recomputes what it needs; a training step can instead keep it from the
 * forward. moe_forward_train is moe_forward (no router options) that also writes, into the
 * caller's `saved` buffer (moe_saved_size bytes, 256-byte aligned, device memory): the float32
 * router logits (T, E), the permutation of the kept slots, and for every kept row the
 * pre-activations x W1 (ReLU, SwiGLU) and x W3 (SwiGLU), the hidden activation and the
 * expert output, in p->dtype. The values are the ones moe_backward recomputes (the same
 * kernels), so moe_backward_saved, given that buffer and the forward's expert_indices, gates,
 * expert_counts, expert_offsets and slot_row, returns bit for bit what moe_backward returns
 * for the same inputs and dout. The caller owns `saved`, must not change it in between, and
 * sizes the workspaces with moe_workspace_size (forward) and moe_backward_workspace_size.
 * Errors as for moe_forward / moe_backward, plus MOE_ERR_WORKSPACE for a missing, short or
 * misaligned `saved` (T > 0). The gradients are the ones moe_backward defines (same passages
 * of the ML Grind and Sparsely-Gated Layer pages). */
size_t moe_saved_size(const moe_problem* p);

moe_status moe_forward_train(const moe_problem* p, const void* x, const void* w_router,
                             const float* router_bias, const void* w1, const void* w3,
                             const void* w2, void* out, int32_t* expert_indices, float* gates,
                             float* aux_loss, int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* slot_row, void* saved, size_t saved_bytes, void* ws,
                             size_t ws_bytes, hipStream_t stream);

moe_status moe_backward_saved(const moe_problem* p, const void* x, const void* w_router,
                              const void* w1, const void* w3, const void* w2,
                              const int32_t* expert_indices, const float* gates,
                              const int32_t* expert_counts, const int32_t* expert_offsets,
                              const int32_t* slot_row, const void* saved, size_t saved_bytes,
                              const void* dout, float d_aux, void* dx, float* dw_router,
                              float* dbias, void* dw1, void* dw3, void* dw2, void* ws,
                              size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* MOE_H */

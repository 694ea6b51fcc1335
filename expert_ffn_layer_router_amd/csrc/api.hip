// The C ABI (include/moe.h): host-side checks, workspace layout, and the launch sequence of
// each entry point. Nothing here allocates memory or synchronises with the device.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.hpp"

using namespace moe;

namespace {

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
size_t elem_size(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

moe_status check_problem(const moe_problem* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (p->kind != MOE_EXPERT_LINEAR && p->kind != MOE_EXPERT_RELU2 && p->kind != MOE_EXPERT_SWIGLU)
    return MOE_ERR_UNSUPPORTED;
  if (p->T < 0 || p->D < 1 || p->D_out < 1 || p->E < 1) return MOE_ERR_INVALID_ARG;
  if (p->kind != MOE_EXPERT_LINEAR && p->DH < 1) return MOE_ERR_INVALID_ARG;
  if (p->top_k < 1 || p->top_k > p->E) return MOE_ERR_INVALID_ARG;
  if (!(p->capacity_factor == p->capacity_factor)) return MOE_ERR_INVALID_ARG;  // NaN
  if (p->E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  // slot and row ids are int32; element offsets are int64
  if (p->T * (int64_t)p->top_k > (int64_t)INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  if (p->D > (int64_t)INT32_MAX || p->D_out > (int64_t)INT32_MAX || p->DH > (int64_t)INT32_MAX)
    return MOE_ERR_UNSUPPORTED;
  if (p->dtype == MOE_BF16) {
    if (p->D % 8 || p->D_out % 8) return MOE_ERR_UNSUPPORTED;
    if (p->kind != MOE_EXPERT_LINEAR && p->DH % 8) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

int64_t capacity_of(const moe_problem* p) {
  if (!(p->capacity_factor > 0.0)) return -1;
  const double c = floor(p->capacity_factor * (double)p->T * (double)p->top_k / (double)p->E);
  if (c >= (double)INT32_MAX) return (int64_t)INT32_MAX;
  return (int64_t)c;
}

Problem internal(const moe_problem* p) {
  Problem q;
  q.T = p->T;
  q.D = p->D;
  q.DH = p->kind == MOE_EXPERT_LINEAR ? 0 : p->DH;
  q.D_out = p->D_out;
  q.E = p->E;
  q.top_k = p->top_k;
  q.capacity = capacity_of(p);
  q.dtype = p->dtype;
  q.kind = p->kind;
  return q;
}

// Byte offsets of every scratch region inside the caller's workspace. `rows` is the number of
// expert-ordered rows: T*k, or with the padded layout max(T*k, E*capacity).
struct Layout {
  int64_t rows;
  size_t route;         // routing scratch (partials, transposed router, partial logits)
  size_t blkc, lrank;   // dispatch: (dispatch blocks, E) int32 and (T*k) int32
  size_t offc;          // padded layout: the compact offsets, (E+1) int32
  size_t hbuf;          // expert hidden activations, (rows, DH)
  size_t gsplit, gctr;  // bf16 GEMM: K-split partial tiles; K-split tickets + work queue
  int64_t nsplit;       // K-split partial tiles reserved (what the layer's GEMMs can use)
  size_t perm;          // moe_forward's own permutation, (rows) int32
  size_t xpad;          // padded layout: the padded copy of x, (rows, D), or one zero row
  size_t ybuf;          // moe_forward's expert outputs, (rows, D_out)
  size_t route_end, dispatch_end, ffn_end, total;
};

// The padded layout's first GEMM gathers x through the padded permutation, its empty rows
// reading one zero row, where the 256 x 256 bf16 kernel runs it (bf16, D % 128 == 0); other
// layers read a padded copy of x.
bool padded_gather(const Problem& q) { return q.dtype == MOE_BF16 && q.D % 128 == 0 && q.T > 0; }

Layout layout_of(const Problem& q, bool padded = false) {
  Layout L;
  L.rows = q.slots();
  if (padded && q.capacity >= 0) L.rows = std::max<int64_t>(L.rows, (int64_t)q.E * q.capacity);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t es = elem_size(q.dtype);
  const size_t slots = (size_t)q.slots();
  const size_t rows = (size_t)L.rows;
  L.route = take(route_ws_bytes(q));
  L.route_end = off;
  L.blkc = take((size_t)dispatch_blocks(q) * q.E * sizeof(int32_t));
  L.lrank = take(slots * sizeof(int32_t));
  L.offc = take(padded ? (size_t)(q.E + 1) * sizeof(int32_t) : 0);
  L.dispatch_end = off;
  L.hbuf = take(q.kind == MOE_EXPERT_LINEAR ? 0 : rows * (size_t)q.DH * es);
  const bool split = q.dtype == MOE_BF16 && q.T > 0;
  // partial tiles for a K split of either GEMM (none when neither K can be split)
  L.nsplit = 0;
  if (split) {
    const bool lin = q.kind == MOE_EXPERT_LINEAR, swi = q.kind == MOE_EXPERT_SWIGLU;
    L.nsplit = gemm_bf16_split_slots(rows, q.E, q.D, lin ? q.D_out : q.DH, swi);
    if (!lin) L.nsplit = std::max(L.nsplit, gemm_bf16_split_slots(rows, q.E, q.DH, q.D_out, false));
  }
  L.gsplit = take((size_t)L.nsplit * kSplitSlotFloats * sizeof(float));
  L.gctr = take(split ? (size_t)(kSplitSlots + kQueueInts) * sizeof(int32_t) : 0);
  L.ffn_end = off;
  L.perm = take(rows * sizeof(int32_t));
  L.xpad = take(padded ? (padded_gather(q) ? 1 : rows) * (size_t)q.D * es : 0);
  L.ybuf = take(rows * (size_t)q.D_out * es);
  L.total = off;
  return L;
}

// Options -> internal form. Noise needs both pointers; the padded layout needs a capacity.
moe_status options_of(const moe_problem* p, const moe_options* o, RouteOpts& ro, bool& padded,
                      float*& importance) {
  ro = RouteOpts{};
  padded = false;
  importance = nullptr;
  if (!o) return MOE_OK;
  if ((o->w_noise == nullptr) != (o->noise == nullptr)) return MOE_ERR_INVALID_ARG;
  ro.w_noise = o->w_noise;
  ro.noise = o->noise;
  ro.renorm = o->no_renormalise == 0;
  padded = o->padded != 0;
  if (padded && capacity_of(p) < 0) return MOE_ERR_INVALID_ARG;
  importance = o->importance_loss;
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MOE_OK;
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

void mark(hipEvent_t* ev, int i, hipStream_t s) {
  if (ev && ev[i]) hipEventRecord(ev[i], s);
}
hipEvent_t event_at(hipEvent_t* ev, int i) { return ev ? ev[i] : nullptr; }

// The expert FFN over expert-ordered rows; `gather` (nullable) maps rows to token rows of A.
// `ev` (nullable) receives the stage markers of the up and down GEMMs.
hipError_t run_experts(const Problem& q, const void* A, const int32_t* gather, const int32_t* offsets,
                       const void* w1, const void* w3, const void* w2, void* hbuf, void* y,
                       void* ws, const Layout& Lw, bool tickets_zeroed, hipStream_t s,
                       hipEvent_t* ev, const void* a_zero = nullptr) {
  const int64_t max_rows = Lw.rows;  // upper bound of offsets[E]
  float* split_ws = nullptr;
  int32_t* split_ctr = nullptr;
  int32_t* queue = nullptr;
  const int ncu = q.dtype == MOE_BF16 ? device_split_cus() : 0;
  if (q.dtype == MOE_BF16 && q.T > 0) {
    int32_t* ctr = at<int32_t>(ws, Lw.gctr);
    queue = ctr + kSplitSlots;
    if (ncu > 0 && Lw.nsplit > 0) {
      split_ws = at<float>(ws, Lw.gsplit);
      split_ctr = ctr;
    }
    // both GEMMs leave the tickets and the queue zero, so one reset before the first serves
    // both
    if (!tickets_zeroed) {
      const hipError_t e0 = launch_zero_tickets(ctr, kSplitSlots + kQueueInts, s);
      if (e0 != hipSuccess) return e0;
    }
  }
  GroupedGemm g{};
  g.split_ws = split_ws;
  g.split_slots = Lw.nsplit;
  g.split_ctr = split_ctr;
  g.ncu = ncu;
  g.queue = queue;
  g.A = A;
  g.lda = q.D;
  g.a_gather = gather;
  g.gather_div = q.top_k;
  g.a_zero = a_zero;
  g.offsets = offsets;
  g.E = q.E;
  g.max_rows = max_rows;
  g.dtype = q.dtype;
  g.K = q.D;
  g.B0 = w1;
  const bool linear = q.kind == MOE_EXPERT_LINEAR;
  g.B1 = (q.kind == MOE_EXPERT_SWIGLU) ? w3 : nullptr;
  g.C = linear ? y : hbuf;
  g.N = linear ? q.D_out : q.DH;
  g.epilogue = linear ? EPI_NONE : (q.kind == MOE_EXPERT_SWIGLU ? EPI_SWIGLU : EPI_RELU);
  // the expert stages' events bracket the GEMM kernels themselves
  g.ev_start = event_at(ev, 2 * MOE_STAGE_EXPERT_UP);
  g.ev_stop = event_at(ev, 2 * MOE_STAGE_EXPERT_UP + 1);
  hipError_t err = launch_grouped_gemm(g, s);
  if (err == hipSuccess && !linear) {
    GroupedGemm d{};
    d.split_ws = split_ws;
    d.split_slots = Lw.nsplit;
    d.split_ctr = split_ctr;
    d.ncu = ncu;
    d.queue = queue;
    d.A = hbuf;
    d.lda = q.DH;
    d.a_gather = nullptr;
    d.gather_div = 1;
    d.B0 = w2;
    d.B1 = nullptr;
    d.C = y;
    d.offsets = offsets;
    d.E = q.E;
    d.K = q.DH;
    d.N = q.D_out;
    d.max_rows = max_rows;
    d.epilogue = EPI_NONE;
    d.dtype = q.dtype;
    d.ev_start = event_at(ev, 2 * MOE_STAGE_EXPERT_DOWN);
    d.ev_stop = event_at(ev, 2 * MOE_STAGE_EXPERT_DOWN + 1);
    err = launch_grouped_gemm(d, s);
  } else {  // no second GEMM: an empty stage
    mark(ev, 2 * MOE_STAGE_EXPERT_DOWN, s);
    mark(ev, 2 * MOE_STAGE_EXPERT_DOWN + 1, s);
  }
  return err;
}

bool weights_ok(const moe_problem* p, const void* w1, const void* w3, const void* w2) {
  if (!w1) return false;
  if (p->kind == MOE_EXPERT_SWIGLU && !w3) return false;
  if (p->kind != MOE_EXPERT_LINEAR && !w2) return false;
  return true;
}

// Routing (launch_route + the loss reduction) with its scratch at `ws` (route_end bytes of the
// layout, 256-byte aligned). Arguments already checked.
moe_status route_into(const Problem& q, const RouteOpts& ro, float* importance, const void* x,
                      const void* w_router, const float* router_bias, int32_t* expert_indices,
                      float* gates, float* aux_loss, int32_t* expert_counts, float* logits_out,
                      int32_t* uncertified, void* route_ws, hipStream_t stream) {
  return hip_status(launch_route_full(q, x, w_router, router_bias, ro, expert_indices, gates,
                                     logits_out, uncertified, aux_loss, expert_counts,
                                     importance, route_ws, stream));
}

moe_status route_args_ok(const moe_problem* p, const void* x, const void* w_router,
                         int32_t* expert_indices, float* gates, float* aux_loss) {
  if (!aux_loss) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!x || !w_router || !expert_indices || !gates)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// ---- the allocation-free routing entry point -------------------------------------------------
// Its scratch is this file-scope device array: each device that loads the library holds its own
// copy until the process ends. In host code `scratch` names a host-side stand-in, so its device
// address is looked up once per device (hipGetSymbolAddress, with that device current) and only
// that address is ever passed to a kernel.
static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_scratch_mu;

// The current device's address of `scratch`; the stream (when not the null stream) must belong
// to that device, since the address is only valid there.
moe_status scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOE_ERR_HIP;
    if ((int)sdev != dev) return MOE_ERR_INVALID_ARG;
  }
  void* ptr = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_dev[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
      g_scratch_dev[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: a null required pointer or a size out of range";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: a shape, dtype or expert kind this library does not handle";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing, too small or not 256-byte aligned";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    case MOE_ERR_SCRATCH_LIMIT:
      return "MOE_ERR_SCRATCH_LIMIT: the problem needs more routing scratch than the "
             "allocation-free entry point's fixed device array (MOE_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown moe_status";
}

moe_status moe_check_problem(const moe_problem* p) { return check_problem(p); }

int64_t moe_capacity(const moe_problem* p) {
  if (check_problem(p) != MOE_OK) return -2;
  return capacity_of(p);
}

size_t moe_workspace_size(const moe_problem* p) {
  if (check_problem(p) != MOE_OK) return 0;
  return layout_of(internal(p)).total;
}

size_t moe_workspace_size_ex(const moe_problem* p, const moe_options* opts) {
  if (check_problem(p) != MOE_OK) return 0;
  RouteOpts ro;
  bool padded;
  float* importance;
  if (options_of(p, opts, ro, padded, importance) != MOE_OK) return 0;
  return layout_of(internal(p), padded).total;
}

moe_status moe_route_ex(const moe_problem* p, const moe_options* opts, const void* x,
                        const void* w_router, const float* router_bias, int32_t* expert_indices,
                        float* gates, float* aux_loss, int32_t* expert_counts,
                        float* logits_out, int32_t* uncertified, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  RouteOpts ro;
  bool padded;
  float* importance;
  st = options_of(p, opts, ro, padded, importance);
  if (st != MOE_OK) return st;
  st = route_args_ok(p, x, w_router, expert_indices, gates, aux_loss);
  if (st != MOE_OK) return st;
  const Problem q = internal(p);
  const Layout L = layout_of(q, padded);
  st = check_ws(ws, ws_bytes, L.route_end);
  if (st != MOE_OK) return st;
  return route_into(q, ro, importance, x, w_router, router_bias, expert_indices, gates, aux_loss,
                    expert_counts, logits_out, uncertified, at<void>(ws, L.route), stream);
}

moe_status moe_route(const moe_problem* p, const void* x, const void* w_router,
                     const float* router_bias, int32_t* expert_indices, float* gates,
                     float* aux_loss, int32_t* expert_counts, float* logits_out,
                     int32_t* uncertified, void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_route_ex(p, nullptr, x, w_router, router_bias, expert_indices, gates, aux_loss,
                      expert_counts, logits_out, uncertified, ws, ws_bytes, stream);
}

moe_status moe_route_noalloc(const moe_problem* p, const void* x, const void* w_router,
                             const float* router_bias, int32_t* expert_indices, float* gates,
                             float* aux_loss, int32_t* expert_counts, float* logits_out,
                             int32_t* uncertified, hipStream_t stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  st = route_args_ok(p, x, w_router, expert_indices, gates, aux_loss);
  if (st != MOE_OK) return st;
  const Problem q = internal(p);
  const Layout L = layout_of(q);
  if (L.route_end > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  st = scratch_of_current_device(stream, &ws);
  if (st != MOE_OK) return st;
  // every counter of the routing scratch is cleared by the routing kernels themselves, so the
  // previous call's contents need no reset here
  return route_into(q, RouteOpts{}, nullptr, x, w_router, router_bias, expert_indices, gates,
                    aux_loss, expert_counts, logits_out, uncertified, at<void>(ws, L.route),
                    stream);
}

moe_status moe_dispatch(const moe_problem* p, const int32_t* expert_indices, const void* x,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                        int32_t* slot_row, void* x_perm, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!expert_offsets) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!expert_indices || !perm || !slot_row)) return MOE_ERR_INVALID_ARG;
  if (x_perm && !x && p->T > 0) return MOE_ERR_INVALID_ARG;
  const Problem q = internal(p);
  const Layout L = layout_of(q);
  st = check_ws(ws, ws_bytes, L.dispatch_end);
  if (st != MOE_OK) return st;
  return hip_status(launch_dispatch(q, expert_indices, x, expert_counts, expert_offsets, perm,
                                    slot_row, x_perm, at<int32_t>(ws, L.blkc),
                                    at<int32_t>(ws, L.lrank), stream));
}

moe_status moe_dispatch_padded(const moe_problem* p, const int32_t* expert_indices,
                               const void* x, int32_t* expert_counts, int32_t* expert_offsets,
                               int32_t* perm, int32_t* slot_row, void* x_pad, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (capacity_of(p) < 0 || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!expert_indices || !slot_row)) return MOE_ERR_INVALID_ARG;
  const Problem q = internal(p);
  if ((int64_t)q.E * q.capacity > 0 && !perm) return MOE_ERR_INVALID_ARG;
  if (x_pad && !x && p->T > 0) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(q, true);
  st = check_ws(ws, ws_bytes, L.dispatch_end);
  if (st != MOE_OK) return st;
  return hip_status(launch_dispatch(q, expert_indices, x, expert_counts,
                                    at<int32_t>(ws, L.offc), perm, slot_row, x_pad,
                                    at<int32_t>(ws, L.blkc), at<int32_t>(ws, L.lrank), stream,
                                    nullptr, 0, expert_offsets));
}

moe_status moe_expert_ffn_ex(const moe_problem* p, const moe_options* opts, const void* x_perm,
                             const int32_t* expert_offsets, const void* w1, const void* w3,
                             const void* w2, void* y_perm, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  RouteOpts ro;
  bool padded;
  float* importance;
  st = options_of(p, opts, ro, padded, importance);
  if (st != MOE_OK) return st;
  if (!expert_offsets || !weights_ok(p, w1, w3, w2)) return MOE_ERR_INVALID_ARG;
  const Problem q = internal(p);
  const Layout L = layout_of(q, padded);
  if (L.rows > 0 && (!x_perm || !y_perm)) return MOE_ERR_INVALID_ARG;
  st = check_ws(ws, ws_bytes, L.ffn_end);
  if (st != MOE_OK) return st;
  if (L.rows == 0) return MOE_OK;
  return hip_status(run_experts(q, x_perm, nullptr, expert_offsets, w1, w3, w2,
                                at<void>(ws, L.hbuf), y_perm, ws, L, false, stream, nullptr));
}

moe_status moe_expert_ffn(const moe_problem* p, const void* x_perm, const int32_t* expert_offsets,
                          const void* w1, const void* w3, const void* w2, void* y_perm, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  return moe_expert_ffn_ex(p, nullptr, x_perm, expert_offsets, w1, w3, w2, y_perm, ws, ws_bytes,
                           stream);
}

moe_status moe_combine(const moe_problem* p, const void* y_perm, const int32_t* slot_row,
                       const float* gates, void* out, hipStream_t stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T > 0 && (!y_perm || !slot_row || !gates || !out)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(internal(p), y_perm, slot_row, gates, out, stream));
}

moe_status moe_forward_ex(const moe_problem* p, const moe_options* opts, const void* x,
                          const void* w_router, const float* router_bias, const void* w1,
                          const void* w3, const void* w2, void* out, int32_t* expert_indices,
                          float* gates, float* aux_loss, int32_t* expert_counts,
                          int32_t* expert_offsets, int32_t* slot_row, void* ws, size_t ws_bytes,
                          hipStream_t stream, hipEvent_t* ev) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  RouteOpts ro;
  bool padded;
  float* importance;
  st = options_of(p, opts, ro, padded, importance);
  if (st != MOE_OK) return st;
  if (!aux_loss || !expert_counts || !expert_offsets || !weights_ok(p, w1, w3, w2))
    return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!x || !w_router || !out || !expert_indices || !gates || !slot_row))
    return MOE_ERR_INVALID_ARG;
  const Problem q = internal(p);
  const Layout L = layout_of(q, padded);
  st = check_ws(ws, ws_bytes, L.total);
  if (st != MOE_OK) return st;
  int32_t* perm = at<int32_t>(ws, L.perm);
  mark(ev, 2 * MOE_STAGE_ROUTE, stream);
  // the fused routing kernel also leaves the offsets and the dispatch ranks' bases (not with
  // the padded layout, whose dispatch has its own kernels)
  bool dispatched = false;
  hipError_t err = launch_route_full(q, x, w_router, router_bias, ro, expert_indices, gates,
                                     nullptr, nullptr, aux_loss, expert_counts, importance,
                                     at<void>(ws, L.route), stream,
                                     padded ? nullptr : expert_offsets,
                                     padded ? nullptr : &dispatched);
  mark(ev, 2 * MOE_STAGE_ROUTE + 1, stream);
  mark(ev, 2 * MOE_STAGE_DISPATCH, stream);
  // the dispatch scan also zeroes the GEMMs' K-split tickets and work queue
  int32_t* tickets = (q.dtype == MOE_BF16 && q.T > 0) ? at<int32_t>(ws, L.gctr) : nullptr;
  const void* A = x;
  const void* a_zero = nullptr;
  const int32_t* gather = perm;
  const int32_t* offsets = expert_offsets;
  if (err == hipSuccess) {
    if (padded) {
      // compact offsets into the workspace and the batch starts into expert_offsets; then
      // either the first GEMM gathers x through the padded permutation (its empty rows, -1,
      // read a zero row), or a padded copy of x is written for it to read row by row
      const bool pg = padded_gather(q);
      err = launch_dispatch(q, expert_indices, x, expert_counts, at<int32_t>(ws, L.offc), perm,
                            slot_row, pg ? nullptr : at<void>(ws, L.xpad),
                            at<int32_t>(ws, L.blkc), at<int32_t>(ws, L.lrank), stream, tickets,
                            tickets ? kSplitSlots + kQueueInts : 0, expert_offsets,
                            pg ? at<void>(ws, L.xpad) : nullptr);
      A = pg ? x : at<void>(ws, L.xpad);
      gather = pg ? perm : nullptr;
      a_zero = pg ? at<void>(ws, L.xpad) : nullptr;
    } else if (dispatched) {
      err = launch_place_after_route(q, expert_indices, at<void>(ws, L.route), aux_loss,
                                     expert_counts, nullptr, expert_offsets, perm, slot_row,
                                     stream, tickets, tickets ? kSplitSlots + kQueueInts : 0,
                                     importance);
    } else {
      err = launch_dispatch(q, expert_indices, x, expert_counts, expert_offsets, perm, slot_row,
                            nullptr, at<int32_t>(ws, L.blkc), at<int32_t>(ws, L.lrank), stream,
                            tickets, tickets ? kSplitSlots + kQueueInts : 0);
    }
  }
  mark(ev, 2 * MOE_STAGE_DISPATCH + 1, stream);
  if (err == hipSuccess)
    err = run_experts(q, A, gather, offsets, w1, w3, w2, at<void>(ws, L.hbuf),
                      at<void>(ws, L.ybuf), ws, L, tickets != nullptr, stream, ev, a_zero);
  mark(ev, 2 * MOE_STAGE_COMBINE, stream);
  if (err == hipSuccess) err = launch_combine(q, at<void>(ws, L.ybuf), slot_row, gates, out, stream);
  mark(ev, 2 * MOE_STAGE_COMBINE + 1, stream);
  return hip_status(err);
}

moe_status moe_forward_timed(const moe_problem* p, const void* x, const void* w_router,
                             const float* router_bias, const void* w1, const void* w3,
                             const void* w2, void* out, int32_t* expert_indices, float* gates,
                             float* aux_loss, int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* slot_row, void* ws, size_t ws_bytes, hipStream_t stream,
                             hipEvent_t* ev) {
  return moe_forward_ex(p, nullptr, x, w_router, router_bias, w1, w3, w2, out, expert_indices,
                        gates, aux_loss, expert_counts, expert_offsets, slot_row, ws, ws_bytes,
                        stream, ev);
}

moe_status moe_forward(const moe_problem* p, const void* x, const void* w_router,
                       const float* router_bias, const void* w1, const void* w3, const void* w2,
                       void* out, int32_t* expert_indices, float* gates, float* aux_loss,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* slot_row,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_forward_ex(p, nullptr, x, w_router, router_bias, w1, w3, w2, out, expert_indices,
                        gates, aux_loss, expert_counts, expert_offsets, slot_row, ws, ws_bytes,
                        stream, nullptr);
}

size_t moe_backward_workspace_size(const moe_problem* p) {
  if (check_problem(p) != MOE_OK) return 0;
  return backward_ws_bytes(internal(p));
}

moe_status moe_backward(const moe_problem* p, const void* x, const void* w_router,
                        const float* router_bias, const void* w1, const void* w3, const void* w2,
                        const void* dout, float d_aux, void* dx, float* dw_router, float* dbias,
                        void* dw1, void* dw3, void* dw2, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!weights_ok(p, w1, w3, w2) || !(d_aux == d_aux)) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!x || !w_router || !dout || !dx || !dw_router || !dw1)) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && p->kind == MOE_EXPERT_SWIGLU && !dw3) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && p->kind != MOE_EXPERT_LINEAR && !dw2) return MOE_ERR_INVALID_ARG;
  const Problem q = internal(p);
  st = check_ws(ws, ws_bytes, backward_ws_bytes(q));
  if (st != MOE_OK) return st;
  if (q.T == 0) return MOE_OK;
  return hip_status(launch_backward(q, x, w_router, router_bias, w1, w3, w2, dout, d_aux, dx,
                                    dw_router, dbias, dw1, dw3, dw2, ws, stream));
}

size_t moe_saved_size(const moe_problem* p) {
  if (check_problem(p) != MOE_OK) return 0;
  return saved_layout(internal(p)).total;
}

moe_status moe_forward_train(const moe_problem* p, const void* x, const void* w_router,
                             const float* router_bias, const void* w1, const void* w3,
                             const void* w2, void* out, int32_t* expert_indices, float* gates,
                             float* aux_loss, int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* slot_row, void* saved, size_t saved_bytes, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!aux_loss || !expert_counts || !expert_offsets || !weights_ok(p, w1, w3, w2))
    return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!x || !w_router || !out || !expert_indices || !gates || !slot_row))
    return MOE_ERR_INVALID_ARG;
  const Problem q = internal(p);
  const Layout L = layout_of(q);
  st = check_ws(ws, ws_bytes, L.total);
  if (st != MOE_OK) return st;
  const SavedLayout S = saved_layout(q);
  st = check_ws(saved, saved_bytes, p->T > 0 ? S.total : 0);
  if (st != MOE_OK) return st;
  char* sv = (char*)saved;
  int32_t* perm = p->T > 0 ? (int32_t*)(sv + S.perm) : at<int32_t>(ws, L.perm);
  bool dispatched = false;
  hipError_t err = launch_route_full(q, x, w_router, router_bias, RouteOpts{}, expert_indices,
                                     gates, p->T > 0 ? (float*)(sv + S.logits) : nullptr, nullptr,
                                     aux_loss, expert_counts, nullptr, at<void>(ws, L.route),
                                     stream, expert_offsets, &dispatched);
  // the dispatch also zeroes the GEMMs' K-split tickets and work queue
  int32_t* tickets = (q.dtype == MOE_BF16 && q.T > 0) ? at<int32_t>(ws, L.gctr) : nullptr;
  if (err == hipSuccess && dispatched)
    err = launch_place_after_route(q, expert_indices, at<void>(ws, L.route), aux_loss,
                                   expert_counts, nullptr, expert_offsets, perm, slot_row, stream,
                                   tickets, tickets ? kSplitSlots + kQueueInts : 0);
  else if (err == hipSuccess)
    err = launch_dispatch(q, expert_indices, x, expert_counts, expert_offsets, perm, slot_row,
                          nullptr, at<int32_t>(ws, L.blkc), at<int32_t>(ws, L.lrank), stream,
                          tickets, tickets ? kSplitSlots + kQueueInts : 0);
  if (err != hipSuccess || q.T == 0) return hip_status(err);
  const int ncu = tickets ? device_split_cus() : 0;
  err = run_experts_saving(q, x, perm, expert_offsets, w1, w3, w2, sv + S.a, sv + S.b, sv + S.h,
                           sv + S.y,
                           (tickets && ncu > 0 && L.nsplit > 0) ? at<float>(ws, L.gsplit) : nullptr,
                           L.nsplit,
                           (tickets && ncu > 0) ? tickets : nullptr,
                           tickets ? tickets + kSplitSlots : nullptr, ncu, stream);
  if (err == hipSuccess) err = launch_combine(q, sv + S.y, slot_row, gates, out, stream);
  return hip_status(err);
}

moe_status moe_backward_saved(const moe_problem* p, const void* x, const void* w_router,
                              const void* w1, const void* w3, const void* w2,
                              const int32_t* expert_indices, const float* gates,
                              const int32_t* expert_counts, const int32_t* expert_offsets,
                              const int32_t* slot_row, const void* saved, size_t saved_bytes,
                              const void* dout, float d_aux, void* dx, float* dw_router,
                              float* dbias, void* dw1, void* dw3, void* dw2, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!weights_ok(p, w1, w3, w2) || !(d_aux == d_aux)) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!x || !w_router || !dout || !dx || !dw_router || !dw1 || !expert_indices ||
                   !gates || !expert_counts || !expert_offsets || !slot_row))
    return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && p->kind == MOE_EXPERT_SWIGLU && !dw3) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && p->kind != MOE_EXPERT_LINEAR && !dw2) return MOE_ERR_INVALID_ARG;
  const Problem q = internal(p);
  st = check_ws(ws, ws_bytes, backward_ws_bytes(q));
  if (st != MOE_OK) return st;
  st = check_ws(saved, saved_bytes, p->T > 0 ? saved_layout(q).total : 0);
  if (st != MOE_OK) return st;
  if (q.T == 0) return MOE_OK;
  return hip_status(launch_backward_saved(q, expert_indices, gates, expert_counts, expert_offsets,
                                          slot_row, saved, x, w_router, w1, w3, w2, dout, d_aux,
                                          dx, dw_router, dbias, dw1, dw3, dw2, ws, stream));
}

}  // extern "C"

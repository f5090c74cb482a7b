// extern "C" entry points of libmoe: validation, workspace layout, launch sequence.
// The computation itself is in router.hip, permute.hip, grouped_mlp.hip and combine.hip.
#include <cmath>
#include <mutex>

#include "common.h"

namespace moe {
namespace {

moe_status to_shape(const moe_config* c, Shape* s) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->reserved != 0) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->n_experts < 1 || c->top_k < 1 || c->top_k > c->n_experts) return MOE_ERR_INVALID_ARG;
  if (c->d_model < 1 || c->d_ff < 1 || c->n_shared < 0) return MOE_ERR_INVALID_ARG;
  if (c->n_shared > 0 && c->d_ff_shared < 1) return MOE_ERR_INVALID_ARG;
  if (c->gating != MOE_SOFTMAX && c->gating != MOE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (c->n_experts > 1024 || c->top_k > 32) return MOE_ERR_UNSUPPORTED;
  if (c->d_model % 64 || c->d_ff % 64) return MOE_ERR_UNSUPPORTED;
  if (c->n_shared > 0 && c->d_ff_shared % 64) return MOE_ERR_UNSUPPORTED;
  if (c->T * static_cast<int64_t>(c->top_k) >= (int64_t{1} << 31)) return MOE_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(c->n_shared) * c->T >= (int64_t{1} << 31)) return MOE_ERR_UNSUPPORTED;
  s->T = c->T;
  s->d = c->d_model;
  s->f = c->d_ff;
  s->E = c->n_experts;
  s->k = c->top_k;
  s->gating = c->gating;
  s->n_shared = c->n_shared;
  s->f_s = c->n_shared > 0 ? c->d_ff_shared : 0;
  s->dtype = c->dtype;
  const double cf = static_cast<double>(c->capacity_factor);
  if (cf > 0) {
    // C = ceil(cf * (T*k) / E) in double precision
    const double cap = std::ceil(cf * static_cast<double>(c->T * c->top_k) / static_cast<double>(c->n_experts));
    if (cap >= 2147483647.0) return MOE_ERR_UNSUPPORTED;
    s->capacity = static_cast<int64_t>(cap);
  } else {
    s->capacity = -1;
  }
  const int64_t pairs = c->T * c->top_k;
  s->max_kept = s->capacity < 0 ? pairs : std::min<int64_t>(pairs, s->capacity * c->n_experts);
  // the tiled GEMMs address rows of one activation matrix (x, h, the shared experts' h)
  // with 32-bit byte offsets: each must stay under 4 GiB
  const int64_t lim = int64_t{1} << 32, esz = c->dtype == MOE_BF16 ? 2 : 4;
  if (s->T * s->d * esz >= lim || s->max_kept * s->f * esz >= lim ||
      static_cast<int64_t>(s->n_shared) * s->T * s->f_s * esz >= lim)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t es(const Shape& s) { return s.dtype == MOE_BF16 ? 2 : 4; }

// Layer workspace: every intermediate of the four steps, 256-byte aligned.
struct LayerWs {
  int32_t* idx;
  float* gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_slot;
  int32_t* pos;
  uint8_t* drop;
  void* permute_ws;
  void* grouped_ws;
  void* y_perm;
  void* y_shared;
  size_t bytes;
};

LayerWs layer_layout(const Shape& s, void* base) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(base);
  size_t off = 0;
  auto take = [&](size_t b) {
    char* r = reinterpret_cast<char*>(p + off);
    off += align256(b);
    return r;
  };
  const size_t pairs = static_cast<size_t>(s.T * s.k);
  LayerWs w;
  w.idx = reinterpret_cast<int32_t*>(take(pairs * 4));
  w.gate = reinterpret_cast<float*>(take(pairs * 4));
  w.counts = reinterpret_cast<int32_t*>(take(static_cast<size_t>(s.E) * 4));
  w.offsets = reinterpret_cast<int32_t*>(take(static_cast<size_t>(s.E + 1) * 4));
  w.sorted_slot = reinterpret_cast<int32_t*>(take(static_cast<size_t>(s.max_kept) * 4));
  w.pos = reinterpret_cast<int32_t*>(take(pairs * 4));
  w.drop = reinterpret_cast<uint8_t*>(take(pairs));
  w.permute_ws = take(permute_ws_bytes(s));
  w.grouped_ws = take(grouped_ws_bytes(s));
  w.y_perm = take(static_cast<size_t>(s.max_kept) * s.d * es(s));
  w.y_shared = take(static_cast<size_t>(s.n_shared) * s.T * s.d * es(s));
  w.bytes = off;
  return w;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The layer workspace's routing and permutation buffers, for a gated launch that routes a
// single token itself (bf16 activations).
RouteArgs route_args(const Shape& s, const void* x, const void* w_router, const float* bias, const LayerWs& w) {
  RouteArgs r;
  r.x = static_cast<const bf16_t*>(x);
  r.w_router = static_cast<const bf16_t*>(w_router);
  r.bias = bias;
  r.idx = w.idx;
  r.gate = w.gate;
  r.counts = w.counts;
  r.offsets = w.offsets;
  r.sorted_slot = w.sorted_slot;
  r.pos = w.pos;
  r.drop = w.drop;
  r.gating = s.gating;
  r.capacity = s.capacity;
  return r;
}

int64_t round64(int64_t v) { return (v + 63) / 64 * 64; }

// K splits of the backward's dx launch (K = 2f, N = d): split while there are fewer than
// four tiles per CU (the last, partly filled round of long-K tiles otherwise dominates)
int bwd_dx_splits(const Shape& s) {
  const int64_t tiles = ((s.d + 255) / 256) * gemm_m_tile_bound(s);
  int sp = 1;
  while (sp < 4 && tiles * sp < 1024 && s.f % (64 * sp) == 0 && (s.n_shared == 0 || s.f_s % (64 * sp) == 0)) sp *= 2;
  return sp;
}

// Backward workspace: the forward's routing state, the recomputed products, the
// intermediates of the dgrad chain, and transposed, zero-padded activations for the weight
// gradients, 256-byte aligned. (The dgrad launches read the weights as stored.)
struct BwdWs {
  int32_t* idx;
  float* gate;
  float* logits;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_slot;
  int32_t* pos;
  uint8_t* drop;
  void* permute_ws;
  int32_t* tiles;
  int32_t* ctrl;  // [0] m-tile count, [16, 64) counters of the six persistent GEMM launches
  void *ab, *ab_s;                  // [rows][2f]: x Wg | x Wu
  void *u, *u_s;                    // [rows][f]: dy Wd
  void *dab, *dab_s, *h, *hs;       // [rows][2f]: da | db;  [rows][f]: h
  float* d_gate;                    // [T*k]
  void* dx_perm;                    // [max_kept][d]
  float* dxpart;                    // split-K partials of the dx launch
  void* dx_s;                       // [n_s + 1][T][d]: shared experts' dx, then the router's
  float* dl;                        // [T][E]
  float* aux_part;                  // [T]
  float* rpart;                     // split-K partials of the router gradients
  int32_t* poff;                    // [E+1]
  void *dypT, *xgT, *hT, *dabT;     // [C][np]: routed segments
  void *dyT, *xT, *hsT, *dabsT;     // [C][tp] ([n_s][C][tp]): shared experts' token rows
  int64_t np, tp;
  size_t bytes;
};

BwdWs bwd_layout(const Shape& s, void* base) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(base);
  size_t off = 0;
  auto take = [&](size_t b) {
    char* r = reinterpret_cast<char*>(p + off);
    off += align256(b);
    return r;
  };
  const size_t pairs = static_cast<size_t>(s.T * s.k);
  const size_t T = static_cast<size_t>(s.T), d = s.d, f = s.f, fs = s.f_s, E = s.E, ns = s.n_shared;
  const size_t mk = static_cast<size_t>(s.max_kept);
  BwdWs w;
  w.np = round64(s.max_kept + 63 * static_cast<int64_t>(s.E));
  w.tp = round64(s.T);
  const size_t np = static_cast<size_t>(w.np), tp = static_cast<size_t>(w.tp);
  w.idx = reinterpret_cast<int32_t*>(take(pairs * 4));
  w.gate = reinterpret_cast<float*>(take(pairs * 4));
  w.logits = reinterpret_cast<float*>(take(T * E * 4));
  w.counts = reinterpret_cast<int32_t*>(take(E * 4));
  w.offsets = reinterpret_cast<int32_t*>(take((E + 1) * 4));
  w.sorted_slot = reinterpret_cast<int32_t*>(take(mk * 4));
  w.pos = reinterpret_cast<int32_t*>(take(pairs * 4));
  w.drop = reinterpret_cast<uint8_t*>(take(pairs));
  w.permute_ws = take(permute_ws_bytes(s));
  w.tiles = reinterpret_cast<int32_t*>(take(static_cast<size_t>(gemm_m_tile_bound(s)) * 4 * 4));
  w.ctrl = reinterpret_cast<int32_t*>(take(64 * 4));
  w.ab = take(mk * 2 * f * 2);
  w.ab_s = take(ns * T * 2 * fs * 2);
  w.u = take(mk * f * 2);
  w.u_s = take(ns * T * fs * 2);
  w.dab = take(mk * 2 * f * 2);
  w.dab_s = take(ns * T * 2 * fs * 2);
  w.h = take(mk * f * 2);
  w.hs = take(ns * T * fs * 2);
  w.d_gate = reinterpret_cast<float*>(take(pairs * 4));
  w.dx_perm = take(mk * d * 2);
  const int dsp = bwd_dx_splits(s);
  w.dxpart = reinterpret_cast<float*>(take(dsp > 1 ? dsp * (mk + ns * T) * d * 4 : 0));
  w.dx_s = take((ns + 1) * T * d * 2);
  w.dl = reinterpret_cast<float*>(take(T * E * 4));
  w.aux_part = reinterpret_cast<float*>(take(T * 4));
  w.rpart = reinterpret_cast<float*>(take(std::max(fma_gemm_ws_bytes(s.E, s.d, s.T), fma_gemm_ws_bytes(s.T, s.d, s.E))));
  w.poff = reinterpret_cast<int32_t*>(take((E + 1) * 4));
  w.dypT = take(d * np * 2);
  w.xgT = take(d * np * 2);
  w.hT = take(f * np * 2);
  w.dabT = take(2 * f * np * 2);
  w.dyT = take(ns ? d * tp * 2 : 0);
  w.xT = take(ns ? d * tp * 2 : 0);
  w.hsT = take(ns * fs * tp * 2);
  w.dabsT = take(ns * 2 * fs * tp * 2);
  w.bytes = off;
  return w;
}

// every matrix a kernel addresses with 32-bit byte offsets stays under 4 GiB
bool bwd_fits_32bit(const Shape& s) {
  const int64_t lim = int64_t{1} << 32;
  const int64_t np = round64(s.max_kept + 63 * static_cast<int64_t>(s.E)), tp = round64(s.T);
  const int64_t wide = std::max<int64_t>(s.d, 2 * static_cast<int64_t>(s.f));
  const int64_t wide_s = std::max<int64_t>(s.d, 2 * static_cast<int64_t>(s.f_s));
  return np * wide * 2 < lim && tp * wide_s * 2 < lim && s.T * static_cast<int64_t>(s.d) * 2 < lim &&
         s.max_kept * 2 * static_cast<int64_t>(s.f) * 2 < lim &&
         static_cast<int64_t>(s.n_shared) * s.T * 2 * s.f_s * 2 < lim;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// FP8 weights: every member present and 16-byte aligned (the kernels read 16-byte vectors
// of codes and of scales)
moe_status check_fp8(const moe_fp8_weights* w) {
  if (!w) return MOE_ERR_INVALID_ARG;
  const void* p[6] = {w->w_gate, w->w_up, w->w_down, w->scale_gate, w->scale_up, w->scale_down};
  for (const void* q : p)
    if (!q || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// the FP8 entry points: bf16 activations, a batch the weight-streaming kernels take, and
// valid weight structs (the shared one only when there are shared experts)
moe_status fp8_args(const Shape& s, const moe_fp8_weights* experts, const moe_fp8_weights* shared,
                    Fp8Scales* sc) {
  if (s.dtype != MOE_BF16 || !small_m_fits(s)) return MOE_ERR_UNSUPPORTED;
  moe_status r = check_fp8(experts);
  if (r == MOE_OK && s.n_shared > 0) r = check_fp8(shared);
  if (r != MOE_OK) return r;
  sc->gate = experts->scale_gate;
  sc->up = experts->scale_up;
  sc->down = experts->scale_down;
  if (s.n_shared > 0) {
    sc->shared_gate = shared->scale_gate;
    sc->shared_up = shared->scale_up;
    sc->shared_down = shared->scale_down;
  }
  return MOE_OK;
}

// Library-owned workspace of moe_layer_forward_noalloc: one copy per GPU, held until the
// process ends. Host code never uses the array's name as an address: the device address of
// each GPU's copy is looked up once, with that device current, and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_WORKSPACE_BYTES];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// the current device's copy of `scratch` (hipGetSymbolAddress on first use on that device)
hipError_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

TimingRequest& timing_request() {
  static thread_local TimingRequest r;
  return r;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: inconsistent configuration or NULL required pointer";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: sizes outside what the kernels tile";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than moe_workspace_size";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a kernel launch failed";
    default: return "unknown moe_status";
  }
}

moe_status moe_check_config(const moe_config* cfg) {
  Shape s;
  return to_shape(cfg, &s);
}

moe_status moe_capacity(const moe_config* cfg, int64_t* capacity) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (!capacity) return MOE_ERR_INVALID_ARG;
  *capacity = s.capacity;
  return MOE_OK;
}

moe_status moe_max_kept(const moe_config* cfg, int64_t* max_kept) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (!max_kept) return MOE_ERR_INVALID_ARG;
  *max_kept = s.max_kept;
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_config* cfg, int op, size_t* bytes) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  switch (op) {
    case MOE_OP_PERMUTE: *bytes = permute_ws_bytes(s); break;
    case MOE_OP_GROUPED_MLP: *bytes = grouped_ws_bytes(s); break;
    case MOE_OP_LAYER: *bytes = layer_layout(s, nullptr).bytes; break;
    case MOE_OP_LAYER_BACKWARD:
      if (s.dtype != MOE_BF16 || !bwd_fits_32bit(s)) return MOE_ERR_UNSUPPORTED;
      *bytes = bwd_layout(s, nullptr).bytes;
      break;
    default: return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* router_bias, int32_t* topk_idx, float* topk_gate, float* logits,
                     void* stream) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (s.T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_route(s, x, w_router, router_bias, topk_idx, topk_gate, logits,
                                 static_cast<hipStream_t>(stream)));
}

moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_slot, int32_t* pos, uint8_t* drop_mask,
                       void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (s.T == 0) return MOE_OK;
  if (!topk_idx || !counts || !offsets || !sorted_slot || !pos || !drop_mask || !ws)
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < permute_ws_bytes(s)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_permute(s, topk_idx, counts, offsets, sorted_slot, pos, drop_mask, ws,
                                   static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_mlp(const moe_config* cfg, const void* x, const int32_t* sorted_slot,
                           const int32_t* offsets, const void* w_gate, const void* w_up,
                           const void* w_down, const void* ws_gate, const void* ws_up,
                           const void* ws_down, void* y_perm, void* y_shared, void* ws,
                           size_t ws_bytes, void* stream) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (s.T == 0) return MOE_OK;
  if (!x || !sorted_slot || !offsets || !w_gate || !w_up || !w_down || !y_perm || !ws)
    return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && (!ws_gate || !ws_up || !ws_down || !y_shared)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < grouped_ws_bytes(s)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_grouped_mlp(s, x, sorted_slot, offsets, w_gate, w_up, w_down, ws_gate,
                                       ws_up, ws_down, y_perm, y_shared, ws,
                                       static_cast<hipStream_t>(stream)));
}

moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* pos,
                       const float* topk_gate, const void* y_shared, void* y, void* stream) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (s.T == 0) return MOE_OK;
  if (!y_perm || !pos || !topk_gate || !y) return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && !y_shared) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(s, y_perm, pos, topk_gate, y_shared, y,
                                   static_cast<hipStream_t>(stream)));
}

moe_status moe_layer_forward(const moe_config* cfg, const void* x, const void* w_router,
                             const float* router_bias, const void* w_gate, const void* w_up,
                             const void* w_down, const void* ws_gate, const void* ws_up,
                             const void* ws_down, void* y, void* ws, size_t ws_bytes,
                             void* stream) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (s.T == 0) return MOE_OK;
  if (!x || !w_router || !w_gate || !w_up || !w_down || !y || !ws) return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && (!ws_gate || !ws_up || !ws_down)) return MOE_ERR_INVALID_ARG;
  LayerWs w = layer_layout(s, ws);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_route_permute(s, x, w_router, router_bias, w.idx, w.gate, nullptr, w.counts, w.offsets,
                                      w.sorted_slot, w.pos, w.drop, w.permute_ws, st);
  if (use_small_m(s)) {
    // small batches: combine straight from the down launch's split-K partials (no y_perm
    // round trip, one launch fewer; the same values as the staged calls); a single token's
    // down launch combines by itself
    SmallCombine comb;
    comb.pos = w.pos;
    comb.gate = w.gate;
    comb.y = y;
    if (e == hipSuccess)
      e = launch_grouped_mlp(s, x, w.sorted_slot, w.offsets, w_gate, w_up, w_down, ws_gate, ws_up,
                             ws_down, nullptr, nullptr, w.grouped_ws, st, Fp8Scales{}, comb);
    if (e == hipSuccess && !small_m_combines(s, false))
      e = launch_combine_partials(s, small_m_partials(s, w.grouped_ws), small_m_splits(s, false), w.pos,
                                  w.gate, y, st);
    return hip_status(e);
  }
  const int sp = large_down_splits(s);
  if (sp > 1) {
    // split-K down launch: combine from its fp32 partials (the same sums and roundings as the
    // reduction into y_perm of the staged calls)
    if (e == hipSuccess)
      e = launch_grouped_mlp(s, x, w.sorted_slot, w.offsets, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, nullptr,
                             nullptr, w.grouped_ws, st);
    if (e == hipSuccess)
      e = launch_combine_partials(s, small_m_partials(s, w.grouped_ws), sp, w.pos, w.gate, y, st);
    return hip_status(e);
  }
  if (e == hipSuccess)
    e = launch_grouped_mlp(s, x, w.sorted_slot, w.offsets, w_gate, w_up, w_down, ws_gate, ws_up,
                           ws_down, w.y_perm, w.y_shared, w.grouped_ws, st);
  if (e == hipSuccess)
    e = launch_combine(s, w.y_perm, w.pos, w.gate, s.n_shared > 0 ? w.y_shared : nullptr, y, st);
  return hip_status(e);
}

moe_status moe_layer_forward_noalloc(const moe_config* cfg, const void* x, const void* w_router,
                                     const float* router_bias, const void* w_gate, const void* w_up,
                                     const void* w_down, const void* ws_gate, const void* ws_up,
                                     const void* ws_down, void* y, void* stream) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (s.T == 0) return MOE_OK;
  if (!x || !w_router || !w_gate || !w_up || !w_down || !y) return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && (!ws_gate || !ws_up || !ws_down)) return MOE_ERR_INVALID_ARG;
  // every check that needs no device comes first: a layer too large for the static buffer is
  // refused before any HIP call
  if (layer_layout(s, nullptr).bytes > static_cast<size_t>(MOE_STATIC_WORKSPACE_BYTES)) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (static_scratch(&ws) != hipSuccess) return MOE_ERR_HIP;
  // the layer's kernels need no part of the workspace zeroed: the persistent GEMM launches'
  // tile counters are cleared by their own tile-table kernel on every call
  return moe_layer_forward(cfg, x, w_router, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y, ws,
                           static_cast<size_t>(MOE_STATIC_WORKSPACE_BYTES), stream);
}

moe_status moe_pack_weights(const moe_config* cfg, const moe_rowvec_weights* src, void* w_router, void* w_gate,
                            void* w_up, void* w_down, void* ws_gate, void* ws_up, void* ws_down, void* stream) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (!src || !src->w_router || !src->w_gate || !src->w_up || !src->w_down) return MOE_ERR_INVALID_ARG;
  if (!w_router || !w_gate || !w_up || !w_down) return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && (!src->ws_gate || !src->ws_up || !src->ws_down || !ws_gate || !ws_up || !ws_down))
    return MOE_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int eb = static_cast<int>(es(s));
  // [d][E] -> [E][d]; [E][d][f] -> [E][f][d]; [E][f][d] -> [E][d][f]
  hipError_t e = launch_transpose_batched(src->w_router, w_router, 1, s.d, s.E, eb, st);
  if (e == hipSuccess) e = launch_transpose_batched(src->w_gate, w_gate, s.E, s.d, s.f, eb, st);
  if (e == hipSuccess) e = launch_transpose_batched(src->w_up, w_up, s.E, s.d, s.f, eb, st);
  if (e == hipSuccess) e = launch_transpose_batched(src->w_down, w_down, s.E, s.f, s.d, eb, st);
  if (s.n_shared > 0) {
    if (e == hipSuccess) e = launch_transpose_batched(src->ws_gate, ws_gate, s.n_shared, s.d, s.f_s, eb, st);
    if (e == hipSuccess) e = launch_transpose_batched(src->ws_up, ws_up, s.n_shared, s.d, s.f_s, eb, st);
    if (e == hipSuccess) e = launch_transpose_batched(src->ws_down, ws_down, s.n_shared, s.f_s, s.d, eb, st);
  }
  return hip_status(e);
}

moe_status moe_expert_shard_forward(const moe_config* cfg, const void* x_recv, const int32_t* local_expert,
                                    const void* w_gate, const void* w_up, const void* w_down, void* y_send,
                                    void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (s.k != 1 || s.capacity >= 0 || s.n_shared != 0) return MOE_ERR_INVALID_ARG;
  if (s.T == 0) return MOE_OK;
  if (!x_recv || !local_expert || !w_gate || !w_up || !w_down || !y_send || !ws) return MOE_ERR_INVALID_ARG;
  LayerWs w = layer_layout(s, ws);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the rows' expert ids are the top-1 choice of a router that ran elsewhere: permute them,
  // run the grouped MLP, and gather each row's output back into receive order (unit gates)
  hipError_t e = launch_permute(s, local_expert, w.counts, w.offsets, w.sorted_slot, w.pos, w.drop, w.permute_ws, st);
  if (use_small_m(s)) {
    if (e == hipSuccess)
      e = launch_grouped_mlp(s, x_recv, w.sorted_slot, w.offsets, w_gate, w_up, w_down, nullptr, nullptr,
                             nullptr, nullptr, nullptr, w.grouped_ws, st);
    if (e == hipSuccess)
      e = launch_combine_partials(s, small_m_partials(s, w.grouped_ws), small_m_splits(s, false), w.pos,
                                  nullptr, y_send, st);
    return hip_status(e);
  }
  const int sp = large_down_splits(s);
  if (sp > 1) {
    if (e == hipSuccess)
      e = launch_grouped_mlp(s, x_recv, w.sorted_slot, w.offsets, w_gate, w_up, w_down, nullptr, nullptr, nullptr,
                             nullptr, nullptr, w.grouped_ws, st);
    if (e == hipSuccess)
      e = launch_combine_partials(s, small_m_partials(s, w.grouped_ws), sp, w.pos, nullptr, y_send, st);
    return hip_status(e);
  }
  if (e == hipSuccess)
    e = launch_grouped_mlp(s, x_recv, w.sorted_slot, w.offsets, w_gate, w_up, w_down, nullptr, nullptr, nullptr,
                           w.y_perm, nullptr, w.grouped_ws, st);
  if (e == hipSuccess) e = launch_combine(s, w.y_perm, w.pos, nullptr, nullptr, y_send, st);
  return hip_status(e);
}

moe_status moe_grouped_mlp_fp8(const moe_config* cfg, const void* x, const int32_t* sorted_slot,
                               const int32_t* offsets, const moe_fp8_weights* experts,
                               const moe_fp8_weights* shared, void* y_perm, void* y_shared, void* ws,
                               size_t ws_bytes, void* stream) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (s.dtype != MOE_BF16 || !small_m_fits(s)) return MOE_ERR_UNSUPPORTED;
  if (s.T == 0) return MOE_OK;
  Fp8Scales sc;
  r = fp8_args(s, experts, shared, &sc);
  if (r != MOE_OK) return r;
  if (!x || !sorted_slot || !offsets || !y_perm || !ws) return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && !y_shared) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < grouped_ws_bytes(s)) return MOE_ERR_WORKSPACE;
  const moe_fp8_weights* sh = s.n_shared > 0 ? shared : nullptr;
  return hip_status(launch_grouped_mlp(s, x, sorted_slot, offsets, experts->w_gate, experts->w_up,
                                       experts->w_down, sh ? sh->w_gate : nullptr, sh ? sh->w_up : nullptr,
                                       sh ? sh->w_down : nullptr, y_perm, y_shared, ws,
                                       static_cast<hipStream_t>(stream), sc));
}

moe_status moe_layer_forward_fp8(const moe_config* cfg, const void* x, const void* w_router,
                                 const float* router_bias, const moe_fp8_weights* experts,
                                 const moe_fp8_weights* shared, void* y, void* ws, size_t ws_bytes,
                                 void* stream) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (s.dtype != MOE_BF16 || !small_m_fits(s)) return MOE_ERR_UNSUPPORTED;
  if (s.T == 0) return MOE_OK;
  Fp8Scales sc;
  r = fp8_args(s, experts, shared, &sc);
  if (r != MOE_OK) return r;
  if (!x || !w_router || !y || !ws) return MOE_ERR_INVALID_ARG;
  LayerWs w = layer_layout(s, ws);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const moe_fp8_weights* sh = s.n_shared > 0 ? shared : nullptr;
  // the small-batch sequence of moe_layer_forward: the combine reads the down launch's
  // split-K partials; a single token is routed inside the gated launch, and its down launch
  // combines by itself
  const RouteArgs route = route_args(s, x, w_router, router_bias, w);
  const bool routes = small_m_routes(s, true);
  SmallCombine comb;
  comb.pos = w.pos;
  comb.gate = w.gate;
  comb.y = y;
  hipError_t e = hipSuccess;
  if (!routes)
    e = launch_route_permute(s, x, w_router, router_bias, w.idx, w.gate, nullptr, w.counts, w.offsets,
                             w.sorted_slot, w.pos, w.drop, w.permute_ws, st);
  if (e == hipSuccess)
    e = launch_grouped_mlp(s, x, w.sorted_slot, w.offsets, experts->w_gate, experts->w_up, experts->w_down,
                           sh ? sh->w_gate : nullptr, sh ? sh->w_up : nullptr, sh ? sh->w_down : nullptr, nullptr,
                           nullptr, w.grouped_ws, st, sc, comb, routes ? &route : nullptr);
  if (e == hipSuccess && !small_m_combines(s, true))
    e = launch_combine_partials(s, small_m_partials(s, w.grouped_ws), small_m_splits(s, false, true), w.pos,
                                w.gate, y, st);
  return hip_status(e);
}

moe_status moe_layer_backward(const moe_config* cfg, const void* x, const void* w_router,
                              const float* router_bias, const void* w_gate, const void* w_up,
                              const void* w_down, const void* ws_gate, const void* ws_up,
                              const void* ws_down, const void* dy, float aux_coef,
                              const moe_layer_grads* g, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  moe_status r = to_shape(cfg, &s);
  if (r != MOE_OK) return r;
  if (!std::isfinite(aux_coef)) return MOE_ERR_INVALID_ARG;
  if (s.dtype != MOE_BF16 || !bwd_fits_32bit(s)) return MOE_ERR_UNSUPPORTED;
  if (s.T == 0) return MOE_OK;
  if (!x || !w_router || !w_gate || !w_up || !w_down || !dy || !g || !ws) return MOE_ERR_INVALID_ARG;
  if (!g->dx || !g->dw_router || !g->dw_gate || !g->dw_up || !g->dw_down) return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && (!ws_gate || !ws_up || !ws_down || !g->dws_gate || !g->dws_up || !g->dws_down))
    return MOE_ERR_INVALID_ARG;
  BwdWs w = bwd_layout(s, ws);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int d = s.d, f = s.f, fs = s.f_s, E = s.E, ns = s.n_shared;
  const int T = static_cast<int>(s.T);
  hipError_t e = launch_fill_u32(w.ctrl, 64, 0, st);
  // forward state: routing, permutation, tile table
  if (e == hipSuccess)
    e = launch_route_permute(s, x, w_router, router_bias, w.idx, w.gate, w.logits, w.counts, w.offsets,
                             w.sorted_slot, w.pos, w.drop, w.permute_ws, st);
  if (e == hipSuccess) e = launch_build_tiles(s, w.offsets, w.tiles, w.ctrl, w.ctrl + 16, st);
  GemmLaunch L{};
  L.tiles = w.tiles;
  L.n_tiles = w.ctrl;
  L.m_bound = gemm_m_tile_bound(s);
  L.E = E;
  L.k = s.k;
  L.T = T;
  L.n_shared = ns;
  L.sorted_slot = w.sorted_slot;
  // (1) recompute a = x Wg and b = x Wu for every kept pair and shared row
  L.mode = kGemmGatedSave;
  L.in_r = L.in_s = x;
  L.w0_r = w_gate;
  L.w1_r = w_up;
  L.w0_s = ws_gate;
  L.w1_s = ws_up;
  L.out_r = w.ab;
  L.out_s = w.ab_s;
  L.N_r = f;
  L.K_r = d;
  L.N_s = fs;
  L.K_s = d;
  L.queue = w.ctrl + 16;
  if (e == hipSuccess) {
    timing_begin(MOE_KERNEL_BWD_RECOMPUTE, st);
    e = launch_grouped_gemm(L, st);
    timing_end(MOE_KERNEL_BWD_RECOMPUTE, st);
  }
  // (2) u = dy Wd: the pair's token row of dy against Wd [d][f] as stored (K = d rows)
  L.mode = kGemmDgradGather;
  L.in_r = L.in_s = dy;
  L.w0_r = w_down;
  L.w1_r = nullptr;
  L.w0_s = ws_down;
  L.w1_s = nullptr;
  L.ksw_r = d;
  L.ksw_s = d;
  L.out_r = w.u;
  L.out_s = w.u_s;
  L.queue = w.ctrl + 24;
  if (e == hipSuccess) {
    timing_begin(MOE_KERNEL_BWD_DOWN_DGRAD, st);
    e = launch_grouped_gemm(L, st);
    timing_end(MOE_KERNEL_BWD_DOWN_DGRAD, st);
  }
  // (3) SwiGLU backward: da | db, h, and each pair's gate gradient u . h
  if (e == hipSuccess) e = launch_fill_u32(w.d_gate, s.T * s.k, 0, st);
  if (e == hipSuccess)
    e = launch_swiglu_bwd(s, w.ab, w.u, w.ab_s, w.u_s, w.offsets, w.sorted_slot, w.gate, w.dab, w.h, w.dab_s, w.hs,
                          w.d_gate, st);
  // (4) dx of every pair: (da | db) against Wg then Wu, [f][d] each as stored (K = 2f rows)
  L.mode = kGemmDgrad;
  L.sorted_slot = nullptr;
  L.in_r = w.dab;
  L.in_s = w.dab_s;
  L.w0_r = w_gate;
  L.w1_r = w_up;
  L.w0_s = ws_gate;
  L.w1_s = ws_up;
  L.ksw_r = f;
  L.ksw_s = fs;
  L.out_r = w.dx_perm;
  L.out_s = w.dx_s;
  L.N_r = d;
  L.K_r = 2 * f;
  L.N_s = d;
  L.K_s = 2 * fs;
  L.queue = w.ctrl + 32;
  const int dsp = bwd_dx_splits(s);
  if (dsp > 1) {  // fp32 partials of the K splits, reduced into dx_perm / dx_s in split order
    L.mode = kGemmDgradSplit;
    L.splits = dsp;
    L.part = w.dxpart;
    L.max_kept = s.max_kept;
  }
  if (e == hipSuccess) {
    timing_begin(MOE_KERNEL_BWD_GATE_UP_DGRAD, st);
    e = launch_grouped_gemm(L, st);
    timing_end(MOE_KERNEL_BWD_GATE_UP_DGRAD, st);
  }
  if (e == hipSuccess && dsp > 1) e = launch_split_reduce(s, w.dxpart, dsp, w.offsets, w.dx_perm, w.dx_s, st);
  // (5) router: logit gradients (+ balancing loss), weight, bias and input gradients
  void* dx_router = static_cast<char*>(w.dx_s) + static_cast<size_t>(ns) * s.T * d * 2;
  if (e == hipSuccess)
    e = launch_router_bwd(s, w.logits, w.idx, w.gate, w.d_gate, w.counts, aux_coef, w.dl, w.aux_part, g->aux_loss,
                          g->d_router_bias, st);
  if (e == hipSuccess) e = launch_fma_gemm(w.dl, 1, E, x, d, E, d, s.T, g->dw_router, d, w.rpart, st);
  if (e == hipSuccess) e = launch_fma_gemm(w.dl, E, 1, w_router, d, s.T, d, E, dx_router, d, w.rpart, st);
  // (6) dx = every kept pair's dx + shared experts' + router's (a combine with unit gates)
  if (e == hipSuccess) {
    Shape s2 = s;
    s2.n_shared = ns + 1;
    e = launch_combine(s2, w.dx_perm, w.pos, nullptr, w.dx_s, g->dx, st);
  }
  // (7) weight gradients over transposed, zero-padded per-expert segments
  if (e == hipSuccess) e = launch_pad_offsets(w.offsets, E, w.poff, st);
  const int np = static_cast<int>(w.np), tp = static_cast<int>(w.tp);
  if (e == hipSuccess)
    e = launch_transpose_segments(dy, d, 0, w.offsets, w.poff, E, 0, w.np, w.sorted_slot, s.k, w.gate, d, w.dypT, np,
                                  0, 1, st);
  if (e == hipSuccess)
    e = launch_transpose_segments(x, d, 0, w.offsets, w.poff, E, 0, w.np, w.sorted_slot, s.k, nullptr, d, w.xgT, np, 0,
                                  1, st);
  if (e == hipSuccess)
    e = launch_transpose_segments(w.h, f, 0, w.offsets, w.poff, E, 0, w.np, nullptr, s.k, nullptr, f, w.hT, np, 0, 1,
                                  st);
  if (e == hipSuccess)
    e = launch_transpose_segments(w.dab, 2 * f, 0, w.offsets, w.poff, E, 0, w.np, nullptr, s.k, nullptr, 2 * f, w.dabT,
                                  np, 0, 1, st);
  if (ns > 0) {
    if (e == hipSuccess)
      e = launch_transpose_segments(dy, d, 0, nullptr, nullptr, 1, T, w.tp, nullptr, s.k, nullptr, d, w.dyT, tp, 0, 1,
                                    st);
    if (e == hipSuccess)
      e = launch_transpose_segments(x, d, 0, nullptr, nullptr, 1, T, w.tp, nullptr, s.k, nullptr, d, w.xT, tp, 0, 1,
                                    st);
    if (e == hipSuccess)
      e = launch_transpose_segments(w.hs, fs, int64_t{T} * fs, nullptr, nullptr, 1, T, w.tp, nullptr, s.k, nullptr, fs,
                                    w.hsT, tp, int64_t{fs} * tp, ns, st);
    if (e == hipSuccess)
      e = launch_transpose_segments(w.dab_s, 2 * fs, int64_t{T} * 2 * fs, nullptr, nullptr, 1, T, w.tp, nullptr, s.k,
                                    nullptr, 2 * fs, w.dabsT, tp, int64_t{2} * fs * tp, ns, st);
  }
  L = GemmLaunch{};
  L.mode = kGemmWgrad;
  L.E = E;
  L.k = s.k;
  L.T = T;
  L.n_shared = ns;
  L.koff = w.poff;
  L.ld_in_r = L.ld_w_r = np;
  L.ld_in_s = L.ld_w_s = tp;
  L.K_s = tp;
  // dWd[e] [d][f] = sum over the segment of (g dy)^T h
  L.in_r = w.dypT;
  L.w0_r = w.hT;
  L.in_s = w.dyT;
  L.in_s_gstride = 0;
  L.w0_s = w.hsT;
  L.w_s_gstride = int64_t{fs} * tp;
  L.M_r = d;
  L.N_r = f;
  L.M_s = d;
  L.N_s = fs;
  L.out_r = g->dw_down;
  L.out_s = g->dws_down;
  L.queue = w.ctrl + 40;
  if (e == hipSuccess) {
    timing_begin(MOE_KERNEL_BWD_DOWN_WGRAD, st);
    e = launch_grouped_gemm(L, st);
    timing_end(MOE_KERNEL_BWD_DOWN_WGRAD, st);
  }
  // dWg[e] [f][d] = da^T x, dWu[e] = db^T x
  L.in_r = w.dabT;
  L.w0_r = w.xgT;
  L.in_s = w.dabsT;
  L.in_s_gstride = int64_t{2} * fs * tp;
  L.w0_s = w.xT;
  L.w_s_gstride = 0;
  L.M_r = f;
  L.N_r = d;
  L.M_s = fs;
  L.N_s = d;
  L.out_r = g->dw_gate;
  L.out_s = g->dws_gate;
  L.queue = w.ctrl + 48;
  if (e == hipSuccess) {
    timing_begin(MOE_KERNEL_BWD_GATE_WGRAD, st);
    e = launch_grouped_gemm(L, st);
    timing_end(MOE_KERNEL_BWD_GATE_WGRAD, st);
  }
  L.in_r = static_cast<const char*>(w.dabT) + static_cast<size_t>(f) * np * 2;
  L.in_s = static_cast<const char*>(w.dabsT) + static_cast<size_t>(fs) * tp * 2;
  L.out_r = g->dw_up;
  L.out_s = g->dws_up;
  L.queue = w.ctrl + 56;
  if (e == hipSuccess) {
    timing_begin(MOE_KERNEL_BWD_UP_WGRAD, st);
    e = launch_grouped_gemm(L, st);
    timing_end(MOE_KERNEL_BWD_UP_WGRAD, st);
  }
  return hip_status(e);
}

moe_status moe_time_next_launch(int kernel, void* begin_event, void* end_event) {
  TimingRequest& r = timing_request();
  if (kernel == -1) {
    r.kernel = -1;
    return MOE_OK;
  }
  if (kernel < MOE_KERNEL_ROUTER || kernel > MOE_KERNEL_BWD_UP_WGRAD || !begin_event || !end_event)
    return MOE_ERR_INVALID_ARG;
  r.kernel = kernel;
  r.begin = static_cast<hipEvent_t>(begin_event);
  r.end = static_cast<hipEvent_t>(end_event);
  return MOE_OK;
}

}  // extern "C"

// extern "C" entry points of libmoe: validation, workspace layout, launch sequence.
// The computation itself is in router.hip, permute.hip, grouped_mlp.hip and combine.hip.
#include <cmath>

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
  if (s.dtype != MOE_BF16 || !use_small_m(s)) return MOE_ERR_UNSUPPORTED;
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
  hipError_t e = launch_route(s, x, w_router, router_bias, w.idx, w.gate, nullptr, st);
  if (e == hipSuccess)
    e = launch_permute(s, w.idx, w.counts, w.offsets, w.sorted_slot, w.pos, w.drop, w.permute_ws, st);
  if (use_small_m(s)) {
    // small batches: combine straight from the down launch's split-K partials (no y_perm
    // round trip, one launch fewer; the same values as the staged calls)
    if (e == hipSuccess)
      e = launch_grouped_mlp(s, x, w.sorted_slot, w.offsets, w_gate, w_up, w_down, ws_gate, ws_up,
                             ws_down, nullptr, nullptr, w.grouped_ws, st);
    if (e == hipSuccess)
      e = launch_combine_partials(s, small_m_partials(s, w.grouped_ws), small_m_splits(s, false), w.pos,
                                  w.gate, y, st);
    return hip_status(e);
  }
  if (e == hipSuccess)
    e = launch_grouped_mlp(s, x, w.sorted_slot, w.offsets, w_gate, w_up, w_down, ws_gate, ws_up,
                           ws_down, w.y_perm, w.y_shared, w.grouped_ws, st);
  if (e == hipSuccess)
    e = launch_combine(s, w.y_perm, w.pos, w.gate, s.n_shared > 0 ? w.y_shared : nullptr, y, st);
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
  if (s.dtype != MOE_BF16 || !use_small_m(s)) return MOE_ERR_UNSUPPORTED;
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
  if (s.dtype != MOE_BF16 || !use_small_m(s)) return MOE_ERR_UNSUPPORTED;
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
  // split-K partials
  hipError_t e = launch_route(s, x, w_router, router_bias, w.idx, w.gate, nullptr, st);
  if (e == hipSuccess)
    e = launch_permute(s, w.idx, w.counts, w.offsets, w.sorted_slot, w.pos, w.drop, w.permute_ws, st);
  if (e == hipSuccess)
    e = launch_grouped_mlp(s, x, w.sorted_slot, w.offsets, experts->w_gate, experts->w_up, experts->w_down,
                           sh ? sh->w_gate : nullptr, sh ? sh->w_up : nullptr, sh ? sh->w_down : nullptr, nullptr,
                           nullptr, w.grouped_ws, st, sc);
  if (e == hipSuccess)
    e = launch_combine_partials(s, small_m_partials(s, w.grouped_ws), small_m_splits(s, false), w.pos, w.gate,
                                y, st);
  return hip_status(e);
}

moe_status moe_time_next_launch(int kernel, void* begin_event, void* end_event) {
  TimingRequest& r = timing_request();
  if (kernel == -1) {
    r.kernel = -1;
    return MOE_OK;
  }
  if (kernel < MOE_KERNEL_ROUTER || kernel > MOE_KERNEL_COMBINE || !begin_event || !end_event)
    return MOE_ERR_INVALID_ARG;
  r.kernel = kernel;
  r.begin = static_cast<hipEvent_t>(begin_event);
  r.end = static_cast<hipEvent_t>(end_event);
  return MOE_OK;
}

}  // extern "C"

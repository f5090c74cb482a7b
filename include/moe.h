/*
 * moe.h -- C ABI of the MI355X (gfx950) Mixture-of-Experts FFN layer forward.
 *
 * One MoE layer on one GPU, in the steps the pages give for it:
 *   router linear layer -> softmax or sigmoid scores -> top-k -> gates renormalised over
 *   the chosen k -> permute tokens by destination expert (dropless, or with a capacity
 *   limit whose overflow is dropped to the residual path) -> each expert's SwiGLU MLP as
 *   a grouped GEMM over its batch (+ optional always-on shared experts) -> undo the
 *   permutation with a gate-weighted combine.
 * Sources: shubhamtatvamasi.com/llm-inference/moe "Mixture of Experts" (sections "The
 * router", "Load imbalance", Q&A "How does a top-k router work?" and "What are capacity
 * factor and token dropping ..."); klaylearn.com/glossary/mixture-of-experts (definition:
 * permute by destination expert, grouped GEMMs per expert batch, undo the permutation);
 * shipai.vats.cc "Mixture of Experts (MoE)" section "How routing works (intuition)".
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except `cfg` and the
 *    out-parameters of moe_workspace_size / moe_capacity, which are host pointers.
 *    The library allocates no memory and keeps no state between calls.
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue work on it:
 *    they are asynchronous, never synchronise the host, and never copy data back.
 *    Calls on different streams with disjoint outputs and workspaces may overlap.
 *    What a call enqueues is kernel launches only (no memset, copy or allocation), so a
 *    call made while `stream` is being captured into a HIP graph replays as part of it,
 *    reading its inputs at replay time.
 *  - Element type of x, every weight, y_perm, y_shared and y is cfg->dtype
 *    (MOE_F32: float; MOE_BF16: bfloat16 bit patterns). Accumulation is fp32.
 *    Router bias and gates are float; indices are int32.
 *  - Layouts are row-major and contiguous. Weights are stored out-features-major, the
 *    layout of a linear layer's weight, i.e. the TRANSPOSE of the d x f matrices of the
 *    row-vector form y = x . W:
 *      x [T][d]   w_router [E][d]   w_gate, w_up [E][f][d]   w_down [E][d][f]
 *      shared: ws_gate, ws_up [n_shared][f_s][d]   ws_down [n_shared][d][f_s]
 *  - Errors are returned before anything is enqueued: MOE_ERR_INVALID_ARG for an
 *    inconsistent config or a NULL required pointer, MOE_ERR_UNSUPPORTED for sizes the
 *    kernels do not tile (see moe_config), MOE_ERR_WORKSPACE for a workspace smaller
 *    than moe_workspace_size. MOE_ERR_HIP reports a failed launch; faults inside a
 *    kernel surface at the caller's next synchronisation. T = 0 is a no-op (MOE_OK).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

enum { MOE_F32 = 0, MOE_BF16 = 1 };       /* moe_config.dtype */
enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 }; /* moe_config.gating */
enum { /* workspace users */
  MOE_OP_PERMUTE = 0,
  MOE_OP_GROUPED_MLP = 1,
  MOE_OP_LAYER = 2,
  MOE_OP_LAYER_BACKWARD = 3
};
enum { /* kernels that moe_time_next_launch can bracket */
  MOE_KERNEL_ROUTER = 0,
  MOE_KERNEL_PERMUTE_SCATTER = 1,
  MOE_KERNEL_GATE_UP = 2, /* grouped gate/up GEMM with the SiLU*mul epilogue */
  MOE_KERNEL_DOWN = 3,    /* grouped down GEMM */
  MOE_KERNEL_COMBINE = 4,
  /* the grouped GEMMs of moe_layer_backward */
  MOE_KERNEL_BWD_RECOMPUTE = 5,     /* x Wg and x Wu of every kept pair, recomputed */
  MOE_KERNEL_BWD_DOWN_DGRAD = 6,    /* u = dy Wd */
  MOE_KERNEL_BWD_GATE_UP_DGRAD = 7, /* dx_pair = da Wg + db Wu */
  MOE_KERNEL_BWD_DOWN_WGRAD = 8,    /* dWd */
  MOE_KERNEL_BWD_GATE_WGRAD = 9,    /* dWg */
  MOE_KERNEL_BWD_UP_WGRAD = 10      /* dWu */
};

/* The problem statement of one layer (the pages' T tokens, d_model, d_ff, E experts,
 * top-k, gating function, capacity factor and shared experts).
 * Limits: 1 <= top_k <= min(E, 32); 1 <= E <= 1024; d_model and d_ff (and d_ff_shared)
 * multiples of 64; T < 2^31 / top_k; each activation matrix under 4 GiB: T*d_model,
 * max_kept*d_ff and n_shared*T*d_ff_shared elements of dtype (MOE_ERR_UNSUPPORTED
 * otherwise). capacity_factor <= 0 means dropless; otherwise each
 * expert keeps at most C = ceil(capacity_factor * T * top_k / E) (token, expert) pairs,
 * the ones with the lowest token index, evaluated in double precision. */
typedef struct moe_config {
  int64_t T;              /* tokens in this call */
  int32_t d_model;        /* d */
  int32_t d_ff;           /* f: width of each routed expert */
  int32_t n_experts;      /* E */
  int32_t top_k;          /* k */
  int32_t gating;         /* MOE_SOFTMAX or MOE_SIGMOID */
  float capacity_factor;  /* <= 0: dropless; must be finite */
  int32_t n_shared;       /* shared experts every token visits (weight 1) */
  int32_t d_ff_shared;    /* f_s (ignored when n_shared == 0) */
  int32_t dtype;          /* MOE_F32 or MOE_BF16 */
  int32_t reserved;       /* must be 0 */
} moe_config;

/* Human-readable name of a status code (static string, never NULL). */
MOE_API const char* moe_status_string(int status);

/* Validates cfg (as every entry point does). */
MOE_API moe_status moe_check_config(const moe_config* cfg);

/* Per-expert capacity C (capacity mode) or -1 (dropless), into *capacity (host). */
MOE_API moe_status moe_capacity(const moe_config* cfg, int64_t* capacity);

/* Upper bound on kept (token, expert) pairs: T*k dropless, min(T*k, E*C) otherwise.
 * This is the row count of sorted_slot and y_perm. Written into *max_kept (host). */
MOE_API moe_status moe_max_kept(const moe_config* cfg, int64_t* max_kept);

/* Bytes of device workspace `op` (MOE_OP_*) needs for cfg, into *bytes (host). */
MOE_API moe_status moe_workspace_size(const moe_config* cfg, int op, size_t* bytes);

/* Router (pages: "The router"; Q&A "How does a top-k router work?").
 *   logits[t][e] = sum_i x[t][i] * w_router[e][i] + router_bias[e]   (fp32 accumulate)
 *   topk_idx[t][j], j < k: the k largest logits, descending, ties to the lower index
 *   (-0 and +0 tie; a NaN logit ranks below every number, so a token whose logits are all
 *   NaN takes experts 0..k-1 and NaN gates: every index is a valid expert);
 *   topk_gate[t][j]: softmax over the chosen logits (= softmax over all E renormalised
 *   over the chosen k), or sigmoid(l) / sum of the chosen sigmoid(l) for MOE_SIGMOID.
 * router_bias [E] float may be NULL (no bias). logits [T][E] float may be NULL. */
MOE_API moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* router_bias, int32_t* topk_idx, float* topk_gate,
                     float* logits, void* stream);

/* Permute (klaylearn "Mixture of Experts" definition; pages' "Load imbalance").
 * Pair s = t*k + j goes to expert topk_idx[s]. Pairs are grouped by expert, and within an
 * expert ordered by ascending token; with a capacity C only the first C of each expert
 * are kept. Outputs (int32 unless noted):
 *   counts[E]          pairs routed to each expert before dropping
 *   offsets[E+1]       exclusive prefix sum of kept pairs; offsets[E] = N_kept
 *   sorted_slot[max_kept]  s of the kept pairs in grouped order; entries >= N_kept are -1
 *   pos[T*k]           index of pair s in the grouped order, -1 if dropped
 *   drop_mask[T*k]     uint8, 1 if pair s was dropped
 * Deterministic (bit-identical on every call). Needs ws of MOE_OP_PERMUTE bytes. */
MOE_API moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_slot, int32_t* pos, uint8_t* drop_mask,
                       void* ws, size_t ws_bytes, void* stream);

/* Grouped expert MLP (klaylearn: one grouped GEMM over the batch of each expert; techbonafide
 * "Experts as Specialized Subnetworks": an expert is a feed-forward block). For every
 * routed expert e and grouped position p in [offsets[e], offsets[e+1]):
 *   v = x[sorted_slot[p] / k];  y_perm[p] = (silu(v . Wg_e) * (v . Wu_e)) . Wd_e
 * and for every shared expert s and token t (pages' "The router": a shared expert runs on
 * every token, without a gate):  y_shared[s][t] = (silu(x_t . Wg_s) * (x_t . Wu_s)) . Wd_s.
 * y_perm [max_kept][d]; y_shared [n_shared][T][d] (required iff n_shared > 0, as are
 * ws_gate/ws_up/ws_down). The intermediate silu(.)*(.) is rounded to dtype.
 * Needs ws of MOE_OP_GROUPED_MLP bytes. */
MOE_API moe_status moe_grouped_mlp(const moe_config* cfg, const void* x, const int32_t* sorted_slot,
                           const int32_t* offsets, const void* w_gate, const void* w_up,
                           const void* w_down, const void* ws_gate, const void* ws_up,
                           const void* ws_down, void* y_perm, void* y_shared, void* ws,
                           size_t ws_bytes, void* stream);

/* Combine (pages' Q&A "How does a top-k router work?": the gate-weighted sum; klaylearn:
 * undo the permutation):
 *   y[t] = sum over j < k with pos[t*k+j] >= 0 of topk_gate[t*k+j] * y_perm[pos[t*k+j]]
 *          + sum over s of y_shared[s][t]
 * in fp32, j ascending, rounded once to dtype. A dropped pair adds nothing (the residual
 * add is the caller's). y_shared may be NULL when n_shared == 0. */
MOE_API moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* pos,
                       const float* topk_gate, const void* y_shared, void* y, void* stream);

/* The whole layer: moe_route, moe_permute, moe_grouped_mlp and moe_combine on one stream,
 * intermediates in ws (MOE_OP_LAYER bytes). y [T][d]. Same results as the four calls. */
MOE_API moe_status moe_layer_forward(const moe_config* cfg, const void* x, const void* w_router,
                             const float* router_bias, const void* w_gate, const void* w_up,
                             const void* w_down, const void* ws_gate, const void* ws_up,
                             const void* ws_down, void* y, void* ws, size_t ws_bytes,
                             void* stream);

/* moe_layer_forward without a workspace argument, for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc. The intermediates live in a workspace the library owns: a static device buffer
 * of MOE_STATIC_WORKSPACE_BYTES (64 MiB) on each GPU the library runs on, held until the
 * process ends. The call allocates nothing (no hipMalloc, no allocating library routine).
 * Layers whose moe_workspace_size(cfg, MOE_OP_LAYER) exceeds the buffer are refused with
 * MOE_ERR_WORKSPACE before anything is enqueued; 64 MiB holds every batch of up to 64 tokens
 * of the Mixtral-, Qwen3- and DeepSeek-V3-shaped layers, and a few hundred tokens of each.
 * All calls on one GPU share that GPU's buffer: calls that overlap on one GPU (other
 * streams, other host threads) race and give undefined results; serialise them. The buffer
 * keeps the last call's contents; nothing in it needs to start at zero.
 * Same arguments, results and errors as moe_layer_forward otherwise. */
#define MOE_STATIC_WORKSPACE_BYTES (64u << 20)
MOE_API moe_status moe_layer_forward_noalloc(const moe_config* cfg, const void* x, const void* w_router,
                                     const float* router_bias, const void* w_gate, const void* w_up,
                                     const void* w_down, const void* ws_gate, const void* ws_up,
                                     const void* ws_down, void* y, void* stream);

/* Weights in the row-vector layout of y = x . W: the d x f matrices as the problem statement
 * writes them (pages: shubhamtatvamasi.com/llm-inference/moe, section "The router": one linear
 * layer maps the token's hidden vector to a logit per expert; klaylearn.com/glossary/
 * mixture-of-experts, definition: each expert is a feed-forward block, run as a grouped GEMM
 * over its batch). Device pointers, row-major, contiguous, element type cfg->dtype:
 *   w_router [d][E]          w_gate, w_up [E][d][f]          w_down [E][f][d]
 *   ws_gate, ws_up [n_shared][d][f_s]                        ws_down [n_shared][f_s][d]
 * (the shared ones only when n_shared > 0). */
typedef struct moe_rowvec_weights {
  const void* w_router;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* ws_gate;
  const void* ws_up;
  const void* ws_down;
} moe_rowvec_weights;

/* One-time pack: writes the weights given in the row-vector layout into the layout every
 * other entry point takes (each matrix transposed: w_router [E][d], w_gate, w_up [E][f][d],
 * w_down [E][d][f], shared [n_shared][f_s][d] and [n_shared][d][f_s]), in buffers the caller
 * owns and then passes to the layer calls. Bit-exact (elements are moved, never rounded).
 * cfg->T is ignored. Sources and destinations must not overlap; all routed pointers are
 * required, the shared ones iff n_shared > 0 (MOE_ERR_INVALID_ARG otherwise). Memory-bound:
 * each weight byte is read and written once. */
MOE_API moe_status moe_pack_weights(const moe_config* cfg, const moe_rowvec_weights* src, void* w_router,
                            void* w_gate, void* w_up, void* w_down, void* ws_gate, void* ws_up,
                            void* ws_down, void* stream);

/* Expert-parallel shard (pages: shubhamtatvamasi.com/llm-inference/moe, section on serving
 * MoE across GPUs: each GPU holds a subset of the experts, token rows are dispatched to the
 * GPU that owns their expert and the expert outputs are sent back to be combined at home;
 * klaylearn "Mixture of Experts" definition: permute by destination expert, grouped GEMM,
 * undo the permutation). The part of one layer step that runs on the GPU owning
 * E_local = cfg->n_experts experts, for the R = cfg->T rows it received:
 *   y_send[r] = (silu(x_recv[r] . Wg_e) * (x_recv[r] . Wu_e)) . Wd_e,  e = local_expert[r]
 * cfg: top_k must be 1, capacity_factor <= 0 (any capacity is applied where the rows are
 * dispatched) and n_shared 0 (shared experts run at home with the home tokens).
 * x_recv [R][d], local_expert [R] int32, y_send [R][d]; w_gate/w_up/w_down hold the local
 * experts only, laid out as for moe_grouped_mlp. Rows keep their order, so the rows received
 * from each source stay one contiguous slice of y_send for the return exchange. A row whose
 * local_expert is outside [0, E_local) is treated as dropped: its y_send row is 0.
 * Each output row is the same computation, in the same order, as that row's y_perm entry
 * in a one-GPU layer whose grouped MLP takes the same kernel path (batches of at most 64
 * rows take the weight-streaming kernels, larger ones the tiled GEMM).
 * Needs ws of MOE_OP_LAYER bytes for cfg. */
MOE_API moe_status moe_expert_shard_forward(const moe_config* cfg, const void* x_recv,
                                    const int32_t* local_expert, const void* w_gate,
                                    const void* w_up, const void* w_down, void* y_send, void* ws,
                                    size_t ws_bytes, void* stream);

/* FP8 expert weights (pages: shubhamtatvamasi.com/llm-inference/moe, "Memory vs compute,
 * quantified": in FP8 the weights take half their BF16 bytes, and small-batch decode time is
 * the time to read the touched experts' weights; shipai.vats.cc "Mixture of Experts (MoE)",
 * table "Production reality: serving MoE is not free": quantising experts is a serving
 * lever whose error differs per expert, so each expert keeps its own scales here).
 * One expert matrix is stored as OCP FP8 E4M3 codes, one byte per element (sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal, 2^-6 * m/8;
 * no infinities; 0x7F and 0xFF are NaN; largest finite value 448), in the layouts of the
 * dtype weights, with one float scale per output row (out feature) of each expert:
 *   W[n][i] = scale[n] * e4m3(code[n][i]).
 * For the routed experts n ranges over E experts and f = d_ff, for the shared experts over
 * n_shared experts and f = d_ff_shared:
 *   w_gate, w_up [n][f][d] codes   w_down [n][d][f] codes
 *   scale_gate, scale_up [n][f]    scale_down [n][d]
 * The struct is a host object; its members are device pointers, all required and 16-byte
 * aligned (MOE_ERR_INVALID_ARG otherwise). Scales are finite; codes are never NaN codes. */
typedef struct moe_fp8_weights {
  const uint8_t* w_gate;
  const uint8_t* w_up;
  const uint8_t* w_down;
  const float* scale_gate;
  const float* scale_up;
  const float* scale_down;
} moe_fp8_weights;

/* moe_grouped_mlp with FP8 expert weights: the same outputs, each weight element being the
 * value it encodes times its row's scale. Activations (x, y_perm, y_shared, the
 * intermediate) stay cfg->dtype, which must be MOE_BF16. Each dot product runs over the
 * exact E4M3 values with an fp32 accumulator; the row's scale multiplies the sum.
 * FP8 weights are meant for decode, where reading the weights is the whole cost: the batch
 * must take the weight-streaming kernels, cfg->T <= 64; larger T, or dtype MOE_F32,
 * returns MOE_ERR_UNSUPPORTED. `shared` (with y_shared) is required when n_shared > 0 and
 * ignored otherwise. Workspace: moe_workspace_size(cfg, MOE_OP_GROUPED_MLP). */
MOE_API moe_status moe_grouped_mlp_fp8(const moe_config* cfg, const void* x, const int32_t* sorted_slot,
                               const int32_t* offsets, const moe_fp8_weights* experts,
                               const moe_fp8_weights* shared, void* y_perm, void* y_shared, void* ws,
                               size_t ws_bytes, void* stream);

/* moe_layer_forward with FP8 expert weights (router weight in cfg->dtype, as before), under
 * the restrictions of moe_grouped_mlp_fp8. The same results as moe_route, moe_permute,
 * moe_grouped_mlp_fp8 and moe_combine called in turn. Workspace: MOE_OP_LAYER bytes. */
MOE_API moe_status moe_layer_forward_fp8(const moe_config* cfg, const void* x, const void* w_router,
                                 const float* router_bias, const moe_fp8_weights* experts,
                                 const moe_fp8_weights* shared, void* y, void* ws, size_t ws_bytes,
                                 void* stream);

/* Gradients written by moe_layer_backward (device pointers, layouts of the inputs they
 * differentiate; element type cfg->dtype unless noted). */
typedef struct moe_layer_grads {
  void* dx;              /* [T][d] */
  void* dw_router;       /* [E][d] */
  float* d_router_bias;  /* [E] float; may be NULL */
  void* dw_gate;         /* [E][f][d] */
  void* dw_up;           /* [E][f][d] */
  void* dw_down;         /* [E][d][f] */
  void* dws_gate;        /* [n_shared][f_s][d]; required iff n_shared > 0 */
  void* dws_up;          /* [n_shared][f_s][d] */
  void* dws_down;        /* [n_shared][d][f_s] */
  float* aux_loss;       /* [1] float: the load-balancing loss value; may be NULL */
} moe_layer_grads;

/* Backward pass of moe_layer_forward (pages: techbonafide.com "Mixture of Experts (MoE)
 * Explained" and klaylearn.com: MoE shapes training as well as inference, and training adds
 * auxiliary losses that keep the experts evenly loaded, after the Switch Transformer work;
 * shipai.vats.cc "Mixture of Experts (MoE)": training adds load-balancing losses;
 * shubhamtatvamasi.com/llm-inference/moe, "The router", "Load imbalance").
 * Given dy [T][d], the gradient of a loss with respect to the layer output y, writes the
 * gradients of  loss + aux_coef * E * sum_e f_e * P_e  with respect to x, the router weight
 * and bias, every routed expert's and every shared expert's weights, where
 *   f_e = (pairs routed to expert e before any capacity drop) / (T * k)   (a constant) and
 *   P_e = mean over tokens of p[t][e], p the router's probability over all E experts:
 *         softmax(logits) for MOE_SOFTMAX, s / sum(s) with s = sigmoid(logits) for MOE_SIGMOID.
 * aux_coef = 0 leaves the balancing loss out. The expert choice and the capacity drop are
 * piecewise constant: no gradient flows through them; dropped pairs contribute nothing.
 * The forward is recomputed inside the call (router, permute, and x Wg, x Wu of every kept
 * pair); the intermediates are rounded to bf16 as in the forward, products accumulate in
 * fp32, and each gradient is rounded once to bf16 (the router's weight and input gradients
 * accumulate in fp32 too). Experts that receive no pairs get zero gradients.
 * cfg->dtype must be MOE_BF16 (MOE_ERR_UNSUPPORTED otherwise, and for shapes whose
 * transposed intermediates exceed 4 GiB per matrix). Needs ws of MOE_OP_LAYER_BACKWARD
 * bytes: activation-sized buffers only (the recomputed products, the dgrad intermediates
 * and transposed activation segments, about 12 * f bytes per kept pair plus a few [T][d]
 * and [kept][d] matrices); the weights are read as stored, never copied. T = 0 writes
 * nothing. */
MOE_API moe_status moe_layer_backward(const moe_config* cfg, const void* x, const void* w_router,
                              const float* router_bias, const void* w_gate, const void* w_up,
                              const void* w_down, const void* ws_gate, const void* ws_up,
                              const void* ws_down, const void* dy, float aux_coef,
                              const moe_layer_grads* grads, void* ws, size_t ws_bytes, void* stream);

/* Instrumentation, for measuring one kernel inside a layer call. The next launch of
 * `kernel` (MOE_KERNEL_*) made by any entry point called on THIS host thread is bracketed
 * by hipEventRecord(begin_event) and hipEventRecord(end_event) on that call's stream;
 * then the request is cleared. begin_event / end_event are hipEvent_t created by the
 * caller. A new request replaces a pending one; kernel = -1 cancels it. */
MOE_API moe_status moe_time_next_launch(int kernel, void* begin_event, void* end_event);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */

// Shared device helpers and the internal launch interface of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/moe.h"

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// fp32 -> bf16, round to nearest even (gfx950 converts in hardware: v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// silu(g) = g * sigmoid(g) with the hardware exp and reciprocal (about 1 ulp each); at
// g -> -inf, exp overflows to inf and the result is -0.
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

__device__ __forceinline__ float sigmoid_f32(float a) { return 1.0f / (1.0f + __expf(-a)); }

// Sums over K splits, in split order from zero, of the float4 at p and the one at p + off2 in
// every split's slice (slices `stride` floats apart). The loads of up to 8 splits are issued
// before any of them is added: split-K partials are written by waves on other XCDs, so every
// load goes past this XCD's L2, and a small batch's reduction otherwise waits on a chain of
// such round trips, one per split.
__device__ __forceinline__ void split_sum2(const float* __restrict__ p, int64_t stride, int64_t off2, int splits,
                                           float4& s0, float4& s1) {
  s0 = make_float4(0.f, 0.f, 0.f, 0.f);
  s1 = s0;
  for (int sp0 = 0; sp0 < splits; sp0 += 8) {
    float4 a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (sp0 + u < splits) {
        const float* q = p + static_cast<int64_t>(sp0 + u) * stride;
        a[u] = *reinterpret_cast<const float4*>(q);
        b[u] = *reinterpret_cast<const float4*>(q + off2);
      }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (sp0 + u < splits) {
        s0.x += a[u].x;
        s0.y += a[u].y;
        s0.z += a[u].z;
        s0.w += a[u].w;
        s1.x += b[u].x;
        s1.y += b[u].y;
        s1.z += b[u].z;
        s1.w += b[u].w;
      }
  }
}

// Internal view of moe_config with derived quantities (host-computed).
struct Shape {
  int64_t T;
  int d, f, E, k, gating, n_shared, f_s, dtype;
  int64_t capacity;  // -1: dropless
  int64_t max_kept;  // rows of sorted_slot / y_perm
};

// Workspace of the permute step: per-chunk expert counts.
constexpr int kPermuteChunk = 1024;  // (token, slot) pairs per chunk (one wave walks one chunk)
int64_t permute_chunks(const Shape& s);
size_t permute_ws_bytes(const Shape& s);

// compute units of the current device (cached per device; 256 if the query fails)
int cu_count();

// Grouped MLP: tile table + intermediate activations.
size_t grouped_ws_bytes(const Shape& s);

// Small batches: the weight-streaming kernels run batches of at most kSmallMMaxRows tokens
// (small_m_fits), the only path for FP8 expert weights. bf16 batches take them while the
// experts average fewer than kSmallMRowsPerExpert rows (T*k < 8E, use_small_m); past that the
// tiled GEMM reads the same weight bytes faster (measured on the Mixtral shape: 0.54 against
// 0.55 ms at T = 32, 0.55 against 0.67 ms at T = 64; the weight-streaming path stays ahead
// at 6 rows per expert and below).
constexpr int kSmallMMaxRows = 64;
constexpr int kSmallMRowsPerExpert = 8;
bool small_m_fits(const Shape& s);
bool use_small_m(const Shape& s);
int small_m_splits(const Shape& s, bool gated, bool fp8 = false);
// K splits of the tiled down launch (1 or 2), from the widths only: a long K against a narrow
// output leaves few tiles per CU, and the last, partly filled round of tiles then dominates
int large_down_splits(const Shape& s);
// y_perm / y_shared from fp32 split partials [splits][max_kept + n_s*T][d], in split order
hipError_t launch_split_reduce(const Shape& s, const float* part, int splits, const int32_t* offsets, void* y_perm,
                               void* y_shared, hipStream_t st);
size_t small_m_ws_bytes(const Shape& s);
// Launches of the bf16 grouped GEMM (grouped_mlp.hip): out[row][n] = sum_k in[src(row)][k] *
// w_g[n][k] over tiles of 256 rows x 256 weight rows.
enum GemmMode {
  kGemmGated = 0,        // forward gate/up with the SiLU*mul epilogue: h [rows][N]
  kGemmPlain = 1,        // forward down: routed rows read in[row], shared rows in[s*T + t]
  kGemmGatedSave = 2,    // gate/up storing both products, [rows][2N] = (x Wg | x Wu)
  kGemmDgradGather = 3,  // one weight matrix stored [K][N], rows read as the gated launch reads them
  kGemmWgrad = 4,        // weight gradients: fixed M rows per group, K = the group's segment
  kGemmPlainSplit = 5,   // kGemmPlain with K split: fp32 partials [splits][max_kept + n_s*T][N]
  kGemmDgrad = 6,        // kGemmPlain rows against weights stored [K][N]: w0 [ksw][N] then w1 [K-ksw][N]
  kGemmDgradSplit = 7    // kGemmDgrad with K split, partials as kGemmPlainSplit
};
struct GemmLaunch {
  int mode;
  const void* in_r;             // routed input
  const void* in_s;             // shared input
  const int32_t* sorted_slot;   // gather of the gated / gather modes
  const int32_t* tiles;         // device tile table (not kGemmWgrad)
  const int32_t* n_tiles;       // device m-tile count (not kGemmWgrad)
  int64_t m_bound;              // bound on m-tiles (grid size)
  const void* w0_r;
  const void* w1_r;
  const void* w0_s;
  const void* w1_s;
  void* out_r;
  void* out_s;
  int N_r, K_r, N_s, K_s;
  int E, k, T, n_shared;
  int32_t* queue;               // 8 zeroed counters
  // kGemmWgrad
  const int32_t* koff;
  int ld_in_r, ld_w_r, ld_in_s, ld_w_s;
  int64_t in_s_gstride, w_s_gstride;
  int M_r, M_s;
  // kGemmPlainSplit, kGemmDgradSplit
  float* part;
  int splits;
  int64_t max_kept;
  // dgrad modes (weights stored [K][N], read along their output index): the first ksw rows
  // of K come from w0 ([E][ksw][N]), the rest from w1 ([E][K-ksw][N]); ksw = K for one matrix
  int ksw_r, ksw_s;
};
hipError_t launch_grouped_gemm(const GemmLaunch& L, hipStream_t st);
// the device tile table of the grouped GEMM (routed groups from offsets, then shared); also
// zeroes 16 queue counters
hipError_t launch_build_tiles(const Shape& s, const int32_t* offsets, int32_t* tiles, int32_t* n_tiles,
                              int32_t* queues, hipStream_t st);
int64_t gemm_m_tile_bound(const Shape& s);

// FP8 (E4M3) expert weights: per-output-row scales of the routed experts, [E][f] (gate, up)
// and [E][d] (down), and of the shared experts, [n_s][f_s] and [n_s][d]; gate null for
// weights in the layer's dtype.
struct Fp8Scales {
  const float* gate = nullptr;
  const float* up = nullptr;
  const float* down = nullptr;
  const float* shared_gate = nullptr;
  const float* shared_up = nullptr;
  const float* shared_down = nullptr;
};

// A single token's routing inputs and outputs (the route + permute launch's), for a gated
// launch that routes the token itself.
struct RouteArgs {
  const bf16_t* x = nullptr;
  const bf16_t* w_router = nullptr;
  const float* bias = nullptr;
  int32_t* idx = nullptr;
  float* gate = nullptr;
  int32_t* counts = nullptr;
  int32_t* offsets = nullptr;
  int32_t* sorted_slot = nullptr;
  int32_t* pos = nullptr;
  uint8_t* drop = nullptr;
  int gating = 0;
  int64_t capacity = -1;
};
// Whether a small-batch step's gated launch routes the batch itself (FP8 expert weights, a
// single token, bf16 activations, E <= 8, its units within 8 waves per CU): then no route launch.
bool small_m_routes(const Shape& s, bool fp8);

// The layer's combine inputs and output, for a down launch that also combines.
struct SmallCombine {
  const int32_t* pos = nullptr;
  const float* gate = nullptr;
  void* y = nullptr;
};
// Whether the down launch of a small-batch step also combines into y (a single token with few
// experts: small_m_down_combine_kernel, or small_m_down_combine_fp8_kernel with FP8 weights),
// given comb.y.
bool small_m_combines(const Shape& s, bool fp8);

// y_perm == nullptr: stop after the down launch and leave the fp32 split-K partials in the
// workspace (small_m_partials) for launch_combine_partials, or, with comb.y set and
// small_m_combines, write y itself
hipError_t launch_grouped_mlp_small(const Shape& s, const void* x, const int32_t* sorted_slot,
                                    const int32_t* offsets, const void* wg, const void* wu,
                                    const void* wd, const void* swg, const void* swu,
                                    const void* swd, void* h, void* hs, float* part,
                                    void* y_perm, void* y_shared, hipStream_t st,
                                    const Fp8Scales& fp8 = Fp8Scales{}, const SmallCombine& comb = SmallCombine{},
                                    const RouteArgs* route = nullptr);
// the down launch's partials [splits][max_kept + n_s*T][d] inside the grouped-MLP workspace
float* small_m_partials(const Shape& s, void* grouped_ws);
// y from the partials: each kept slot's row is summed over the splits in order and rounded
// to bf16 exactly as the reduction into y_perm does, then combined as launch_combine does
hipError_t launch_combine_partials(const Shape& s, const float* part, int splits, const int32_t* pos,
                                   const float* gate, void* y, hipStream_t st);

// Launchers (return hipSuccess or the launch error).
hipError_t launch_route(const Shape& s, const void* x, const void* w_router, const float* bias,
                        int32_t* idx, float* gate, float* logits, hipStream_t st);
hipError_t launch_permute(const Shape& s, const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_slot, int32_t* pos, uint8_t* drop, void* ws,
                          hipStream_t st);
// launch_route then launch_permute, as one launch when both fit one block (small batches);
// the same results either way
hipError_t launch_route_permute(const Shape& s, const void* x, const void* w_router, const float* bias,
                                int32_t* idx, float* gate, float* logits, int32_t* counts, int32_t* offsets,
                                int32_t* sorted_slot, int32_t* pos, uint8_t* drop, void* permute_ws,
                                hipStream_t st);
// fp8: scales of FP8 expert weights (the weight-streaming path only: the caller checks small_m_fits)
hipError_t launch_grouped_mlp(const Shape& s, const void* x, const int32_t* sorted_slot,
                              const int32_t* offsets, const void* wg, const void* wu,
                              const void* wd, const void* swg, const void* swu, const void* swd,
                              void* y_perm, void* y_shared, void* ws, hipStream_t st,
                              const Fp8Scales& fp8 = Fp8Scales{}, const SmallCombine& comb = SmallCombine{},
                              const RouteArgs* route = nullptr);
hipError_t launch_combine(const Shape& s, const void* y_perm, const int32_t* pos,
                          const float* gate, const void* y_shared, void* y, hipStream_t st);

// Backward pass (backward.hip).
hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* poff, hipStream_t st);
hipError_t launch_transpose_segments(const void* src, int src_ld, int64_t src_bstride, const int32_t* off,
                                     const int32_t* poff, int nseg, int len1, int64_t padded_rows_bound,
                                     const int32_t* sorted_slot, int k, const float* gate, int C, void* dst, int ldd,
                                     int64_t dst_bstride, int batch, hipStream_t st);
hipError_t launch_swiglu_bwd(const Shape& s, const void* ab, const void* u, const void* ab_s, const void* u_s,
                             const int32_t* offsets, const int32_t* sorted_slot, const float* gate, void* dab, void* h,
                             void* dab_s, void* hs, float* d_gate, hipStream_t st);
hipError_t launch_router_bwd(const Shape& s, const float* logits, const int32_t* idx, const float* gate,
                             const float* d_gate, const int32_t* counts, float aux_coef, float* dl, float* aux_part,
                             float* aux_loss, float* d_bias, hipStream_t st);
// split-K over ~1024 blocks when M x N is small; partials: fma_gemm_ws_bytes of fp32
size_t fma_gemm_ws_bytes(int64_t M, int N, int64_t K);
hipError_t launch_fma_gemm(const float* A, int64_t sam, int64_t sak, const void* B, int64_t ldb, int64_t M, int N,
                           int64_t K, void* C, int64_t ldc, float* partials, hipStream_t st);
hipError_t launch_fill_u32(void* p, int64_t n, uint32_t v, hipStream_t st);

// Weight pack (pack.hip): dst[b][c][r] = src[b][r][c] for `batch` R x C matrices of 2- or
// 4-byte elements.
hipError_t launch_transpose_batched(const void* src, void* dst, int64_t batch, int R, int C, int elem_bytes,
                                    hipStream_t st);

struct TimingRequest {
  int kernel = -1;
  hipEvent_t begin = nullptr, end = nullptr;
};
TimingRequest& timing_request();
inline void timing_begin(int kernel, hipStream_t st) {
  TimingRequest& r = timing_request();
  if (r.kernel == kernel) (void)hipEventRecord(r.begin, st);
}
inline void timing_end(int kernel, hipStream_t st) {
  TimingRequest& r = timing_request();
  if (r.kernel == kernel) {
    (void)hipEventRecord(r.end, st);
    r.kernel = -1;
  }
}

inline size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace moe

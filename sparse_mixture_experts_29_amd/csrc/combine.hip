// Combine: undo the permutation and take the gate-weighted sum of each token's kept
// expert outputs, plus every shared expert's output.
// Pages: shubhamtatvamasi.com/llm-inference/moe, Q&A "How does a top-k router work?" (the
// token's output is the gate-weighted sum of its experts' outputs) and section "Load
// imbalance" (a dropped pair skips its expert: it contributes nothing here);
// klaylearn.com/glossary/mixture-of-experts, definition (the last step reverses the permutation).
//
// gate == nullptr means unit gates (the expert-parallel shard returns each row's output).
// A gather, not a scatter: each block owns tokens and reads their k rows of y_perm, so
// the fp32 sum runs in a fixed order (j ascending, then shared experts) and is
// bit-reproducible. Each thread handles 8 consecutive elements (16 B of bf16).
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <typename T>
struct Vec8;
template <>
struct Vec8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
    const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r[i] << 16);
      v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4*>(p) = r;
  }
};
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// grid: ceil(T / tokens_per_block); each token's d/8 chunks are spread over the block.
template <typename T>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const T* __restrict__ y_perm, const int32_t* __restrict__ pos, const float* __restrict__ gate,
    const T* __restrict__ y_shared, T* __restrict__ y, int64_t n_tok, int d, int k, int n_shared,
    int tok_per_block) {
  const int chunks = d / 8;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tok_per_block;
  for (int i = threadIdx.x; i < tok_per_block * chunks; i += kThreads) {
    const int64_t t = t0 + i / chunks;
    const int c = i % chunks;
    if (t >= n_tok) break;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // slots in groups of 8: positions and gates first, then every row load of the group
    // issued before any is used (a dropped slot reads row 0, which exists whenever T >= 1,
    // and is discarded), then the sum in slot order, as if dropped slots were skipped
    for (int j0 = 0; j0 < k; j0 += 8) {
      int pj[8];
      float gj[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool in = j0 + q < k;
        pj[q] = in ? pos[t * k + j0 + q] : -1;
        gj[q] = in ? (gate ? gate[t * k + j0 + q] : 1.f) : 0.f;
      }
      float v[8][8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        Vec8<T>::load(y_perm + static_cast<int64_t>(pj[q] >= 0 ? pj[q] : 0) * d + c * 8, v[q]);
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = pj[q] >= 0 ? fmaf(gj[q], v[q][u], acc[u]) : acc[u];
    }
    for (int s = 0; s < n_shared; ++s) {
      float v[8];
      Vec8<T>::load(y_shared + (static_cast<int64_t>(s) * n_tok + t) * d + c * 8, v);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += v[u];
    }
    Vec8<T>::store(y + t * d + c * 8, acc);
  }
}

// Row chunk c of partial row `row`: the sum over the splits in split order, rounded to
// bf16 and widened back (the value the ordered reduction stores into y_perm).
__device__ __forceinline__ void split_sum_bf16(const float* __restrict__ part, int64_t row, int64_t rows_total,
                                               int d, int c, int splits, float* v) {
  float4 s0, s1;
  split_sum2(part + row * d + c * 8, rows_total * d, 4, splits, s0, s1);
  const uint32_t w[4] = {pack_bf16x2(s0.x, s0.y), pack_bf16x2(s0.z, s0.w), pack_bf16x2(s1.x, s1.y),
                         pack_bf16x2(s1.z, s1.w)};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Small-batch layer: combine straight from the down launch's split-K partials (rows
// [0, max_kept) routed, then max_kept + s*T + t for shared expert s), skipping the bf16
// y_perm round trip; same arithmetic, same order as reduce + combine_kernel.
__global__ __launch_bounds__(kThreads) void combine_partials_kernel(
    const float* __restrict__ part, int splits, int64_t max_kept, const int32_t* __restrict__ pos,
    const float* __restrict__ gate, bf16_t* __restrict__ y, int64_t n_tok, int d, int k, int n_shared) {
  const int chunks = d / 8;
  const int64_t rows_total = max_kept + static_cast<int64_t>(n_shared) * n_tok;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n_tok * chunks) return;
  const int64_t t = i / chunks;
  const int c = static_cast<int>(i % chunks);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int p = pos[t * k + j];
    if (p < 0) continue;
    const float g = gate ? gate[t * k + j] : 1.f;
    float v[8];
    split_sum_bf16(part, p, rows_total, d, c, splits, v);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = fmaf(g, v[u], acc[u]);
  }
  for (int s = 0; s < n_shared; ++s) {
    float v[8];
    split_sum_bf16(part, max_kept + static_cast<int64_t>(s) * n_tok + t, rows_total, d, c, splits, v);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += v[u];
  }
  Vec8<bf16_t>::store(y + t * d + c * 8, acc);
}

}  // namespace

hipError_t launch_combine_partials(const Shape& s, const float* part, int splits, const int32_t* pos,
                                   const float* gate, void* y, hipStream_t st) {
  const int64_t threads = s.T * (s.d / 8);
  timing_begin(MOE_KERNEL_COMBINE, st);
  hipLaunchKernelGGL(combine_partials_kernel, dim3(static_cast<unsigned>((threads + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, part, splits, s.max_kept, pos, gate, static_cast<bf16_t*>(y), s.T,
                     s.d, s.k, s.n_shared);
  timing_end(MOE_KERNEL_COMBINE, st);
  return hipGetLastError();
}

hipError_t launch_combine(const Shape& s, const void* y_perm, const int32_t* pos,
                          const float* gate, const void* y_shared, void* y, hipStream_t st) {
  const int chunks = s.d / 8;
  const int tpb = chunks >= kThreads ? 1 : kThreads / chunks;
  const dim3 grid(static_cast<unsigned>((s.T + tpb - 1) / tpb));
  timing_begin(MOE_KERNEL_COMBINE, st);
  if (s.dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(kThreads), 0, st,
                       static_cast<const bf16_t*>(y_perm), pos, gate,
                       static_cast<const bf16_t*>(y_shared), static_cast<bf16_t*>(y), s.T, s.d,
                       s.k, s.n_shared, tpb);
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(kThreads), 0, st,
                       static_cast<const float*>(y_perm), pos, gate,
                       static_cast<const float*>(y_shared), static_cast<float*>(y), s.T, s.d, s.k,
                       s.n_shared, tpb);
  timing_end(MOE_KERNEL_COMBINE, st);
  return hipGetLastError();
}

}  // namespace moe

// Permute: group the (token, slot) pairs by destination expert, stable in token order,
// with an optional per-expert capacity that drops the overflow.
// Pages: klaylearn.com/glossary/mixture-of-experts, definition (tokens are regrouped
// by the expert they go to); shubhamtatvamasi.com/llm-inference/moe, section "Load imbalance"
// (capacity factor x ideal tokens; overflow skips the expert) and Q&A on capacity factor
// (limit factor x (T.k/E)); dropless when no capacity is set.
//
// Pair s = t*k + j. Each token picks an expert at most once, so ascending s within an
// expert is ascending token order, and "keep the lowest tokens" is "keep rank < C".
// An expert id outside [0, E) (possible only in rows handed to moe_expert_shard_forward)
// marks its pair dropped; it is never used as an index.
// Three launches (one, permute_single_kernel, when the pairs fit one chunk), all
// deterministic (no order-dependent atomics):
//   1. hist:    per chunk of 1024 pairs, a per-expert count (LDS counters).
//   2. scan:    one block; per expert, exclusive prefix over chunks (chunk bases), the
//               expert totals (counts), capped totals, and offsets = their prefix sum.
//   3. scatter: per chunk; each wave ranks its 256 pairs in 4 rounds of 64 lanes, equal
//               experts found with ballots over the expert id bits; rank = chunk base +
//               earlier waves + earlier rounds + earlier lanes.
#include "permute_block.h"

namespace moe {
namespace {

constexpr int kThreads = kPermuteThreads;

__global__ __launch_bounds__(kThreads) void permute_hist_kernel(const int32_t* __restrict__ idx,
                                                                int64_t n_pairs, int E,
                                                                int32_t* __restrict__ chunk_cnt) {
  extern __shared__ int cnt[];
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kPermuteChunk;
  for (int i = threadIdx.x; i < kPermuteChunk; i += kThreads) {
    const int64_t s = s0 + i;
    if (s < n_pairs) {
      const int e = idx[s];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads)
    chunk_cnt[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
}

constexpr int kScanThreads = 1024;

// One block. Thread layout: G groups of chunks per expert (G * Epad <= 1024).
__global__ __launch_bounds__(kScanThreads) void permute_scan_kernel(
    int32_t* __restrict__ chunk_cnt, int n_chunks, int E, int Epad, int64_t capacity,
    int64_t max_kept, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slot) {
  __shared__ int part[kScanThreads];
  __shared__ int kept_scan[kScanThreads];
  const int G = kScanThreads / Epad;
  const int e = threadIdx.x % Epad, g = threadIdx.x / Epad;
  const int per = (n_chunks + G - 1) / G;
  const int c0 = g * per, c1 = min(n_chunks, c0 + per);
  int sum = 0;
  if (e < E)
    for (int c = c0; c < c1; ++c) sum += chunk_cnt[static_cast<int64_t>(c) * E + e];
  part[threadIdx.x] = sum;
  __syncthreads();
  // prefix over the groups of the same expert
  int before = 0, total = 0;
  for (int gg = 0; gg < G; ++gg) {
    const int v = part[gg * Epad + e];
    if (gg < g) before += v;
    total += v;
  }
  if (e < E) {
    int run = before;
    for (int c = c0; c < c1; ++c) {
      const int64_t o = static_cast<int64_t>(c) * E + e;
      const int v = chunk_cnt[o];
      chunk_cnt[o] = run;  // chunk base: pairs of expert e in earlier chunks
      run += v;
    }
  }
  // per-expert totals, capped totals and their exclusive prefix (offsets)
  int kept = 0;
  if (g == 0 && e < E) {
    counts[e] = total;
    kept = (capacity >= 0 && total > capacity) ? static_cast<int>(capacity) : total;
  }
  __syncthreads();
  kept_scan[threadIdx.x] = (g == 0) ? kept : 0;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {  // Hillis-Steele inclusive scan
    const int v = threadIdx.x >= off ? kept_scan[threadIdx.x - off] : 0;
    __syncthreads();
    kept_scan[threadIdx.x] += v;
    __syncthreads();
  }
  if (g == 0 && e < E) offsets[e] = kept_scan[e] - kept;
  const int n_kept = kept_scan[Epad - 1];
  if (threadIdx.x == 0) offsets[E] = n_kept;
  for (int64_t p = n_kept + threadIdx.x; p < max_kept; p += kScanThreads) sorted_slot[p] = -1;
}

__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t n_pairs, int E, int ebits, int64_t capacity,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ pos, uint8_t* __restrict__ drop) {
  extern __shared__ int lds[];
  int* wbase = lds;  // [4][E]: rank base of each wave, per expert
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t s_wave = static_cast<int64_t>(blockIdx.x) * kPermuteChunk + wave * 256;
  for (int i = threadIdx.x; i < 4 * E; i += kThreads) wbase[i] = 0;
  __syncthreads();
  int ex[kPairsPerThread];
#pragma unroll
  for (int r = 0; r < kPairsPerThread; ++r) {
    const int64_t s = s_wave + r * 64 + lane;
    ex[r] = s < n_pairs ? idx[s] : -1;
    if (static_cast<unsigned>(ex[r]) >= static_cast<unsigned>(E)) {
      if (s < n_pairs) {  // an expert id outside [0, E): the pair is dropped
        pos[s] = -1;
        drop[s] = 1;
      }
      ex[r] = -1;
    }
    if (ex[r] >= 0) atomicAdd(&wbase[wave * E + ex[r]], 1);
  }
  __syncthreads();
  // turn per-wave counts into bases: chunk base + counts of earlier waves
  for (int e = threadIdx.x; e < E; e += kThreads) {
    int run = chunk_base[static_cast<int64_t>(blockIdx.x) * E + e];
    for (int w = 0; w < 4; ++w) {
      const int v = wbase[w * E + e];
      wbase[w * E + e] = run;
      run += v;
    }
  }
  __syncthreads();
  rank_and_write(ex, wbase + wave * E, s_wave, ebits, capacity, offsets, sorted_slot, pos, drop);
}

// All three steps in one block when the pairs fit one chunk (small batches).
__global__ __launch_bounds__(kThreads) void permute_single_kernel(
    const int32_t* __restrict__ idx, int64_t n_pairs, int E, int ebits, int64_t capacity,
    int64_t max_kept, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ pos, uint8_t* __restrict__ drop) {
  extern __shared__ int lds[];
  permute_single_block(idx, n_pairs, E, ebits, capacity, max_kept, counts, offsets, sorted_slot, pos, drop, lds);
}

}  // namespace

int64_t permute_chunks(const Shape& s) {
  return (s.T * s.k + kPermuteChunk - 1) / kPermuteChunk;
}

size_t permute_ws_bytes(const Shape& s) {
  return align256(static_cast<size_t>(permute_chunks(s)) * s.E * sizeof(int32_t));
}

hipError_t launch_permute(const Shape& s, const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_slot, int32_t* pos, uint8_t* drop, void* ws,
                          hipStream_t st) {
  const int64_t n_pairs = s.T * s.k;
  const int n_chunks = static_cast<int>(permute_chunks(s));
  int ebits = 0;
  while ((1 << ebits) < s.E) ++ebits;
  if (n_chunks == 1) {
    timing_begin(MOE_KERNEL_PERMUTE_SCATTER, st);
    hipLaunchKernelGGL(permute_single_kernel, dim3(1), dim3(kThreads), (5 * s.E + 1 + kThreads) * sizeof(int), st,
                       idx, n_pairs, s.E, ebits, s.capacity, s.max_kept, counts, offsets, sorted_slot, pos, drop);
    timing_end(MOE_KERNEL_PERMUTE_SCATTER, st);
    return hipGetLastError();
  }
  int32_t* chunk_cnt = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(permute_hist_kernel, dim3(n_chunks), dim3(kThreads), s.E * sizeof(int), st,
                     idx, n_pairs, s.E, chunk_cnt);
  int Epad = 1;
  while (Epad < s.E) Epad <<= 1;
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kScanThreads), 0, st, chunk_cnt, n_chunks,
                     s.E, Epad, s.capacity, s.max_kept, counts, offsets, sorted_slot);
  timing_begin(MOE_KERNEL_PERMUTE_SCATTER, st);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(n_chunks), dim3(kThreads), 4 * s.E * sizeof(int),
                     st, idx, n_pairs, s.E, ebits, s.capacity, chunk_cnt, offsets, sorted_slot, pos,
                     drop);
  timing_end(MOE_KERNEL_PERMUTE_SCATTER, st);
  return hipGetLastError();
}

}  // namespace moe

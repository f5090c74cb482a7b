// One-block permute, shared by the permute launch for small batches and the fused route +
// permute kernel: per-wave expert counts in LDS, expert totals, capped totals and their prefix
// (offsets), then a stable rank of every pair within its expert (ballots over the expert id
// bits), so the result is the scatter's with chunk base 0.
// Pages: klaylearn.com/glossary/mixture-of-experts, definition (tokens regrouped by the expert
// they go to); shubhamtatvamasi.com/llm-inference/moe, section "Load imbalance" (capacity:
// the overflow skips the expert).
#ifndef MOE_PERMUTE_BLOCK_H_
#define MOE_PERMUTE_BLOCK_H_

#include "common.h"

namespace moe {
namespace {

constexpr int kPermuteThreads = 256;
constexpr int kPairsPerThread = kPermuteChunk / kPermuteThreads;  // 4

// Ranks and writes the wave's pairs ex[r] (pair s_wave + 64 r + lane; -1 = none): `base`
// [E] holds, per expert, the rank of the wave's first pair and is advanced as it goes.
__device__ __forceinline__ void rank_and_write(const int (&ex)[kPairsPerThread], int* base, int64_t s_wave,
                                               int ebits, int64_t capacity, const int32_t* offsets,
                                               int32_t* __restrict__ sorted_slot, int32_t* __restrict__ pos,
                                               uint8_t* __restrict__ drop) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int r = 0; r < kPairsPerThread; ++r) {
    const int e = ex[r];
    const bool valid = e >= 0;
    // lanes holding the same expert id
    uint64_t same = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    int rank = 0;
    if (valid) {
      const int before = __popcll(same & lt_mask);
      rank = base[e] + before;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (valid && (same >> lane) == 1ull)  // highest lane of the group advances the base
      base[e] += __popcll(same);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      const int64_t s = s_wave + r * 64 + lane;
      if (capacity < 0 || rank < capacity) {
        const int p = offsets[e] + rank;
        sorted_slot[p] = static_cast<int32_t>(s);
        pos[s] = p;
        drop[s] = 0;
      } else {
        pos[s] = -1;
        drop[s] = 1;
      }
    }
  }
}

// LDS ints the one-block permute needs for E experts
constexpr int permute_block_lds_ints(int E) { return 5 * E + 1 + kPermuteThreads; }

// All three permute steps by one block of kPermuteThreads threads, for n_pairs <= kPermuteChunk
// pairs; lds holds permute_block_lds_ints(E) ints.
__device__ __forceinline__ void permute_single_block(
    const int32_t* __restrict__ idx, int64_t n_pairs, int E, int ebits, int64_t capacity,
    int64_t max_kept, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ pos, uint8_t* __restrict__ drop, int* lds) {
  int* wbase = lds;              // [4][E]
  int* off = lds + 4 * E;        // [E + 1]: offsets
  int* scan = off + E + 1;       // [kPermuteThreads]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t s_wave = wave * 256;
  for (int i = threadIdx.x; i < 4 * E; i += kPermuteThreads) wbase[i] = 0;
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
  // thread i owns experts [4i, 4i+4) (E <= 1024): totals, wave bases, capped totals
  int kept4[4], local = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x * 4 + q;
    kept4[q] = 0;
    if (e < E) {
      int run = 0;
      for (int w = 0; w < 4; ++w) {
        const int v = wbase[w * E + e];
        wbase[w * E + e] = run;
        run += v;
      }
      counts[e] = run;
      kept4[q] = (capacity >= 0 && run > capacity) ? static_cast<int>(capacity) : run;
    }
    local += kept4[q];
  }
  scan[threadIdx.x] = local;
  __syncthreads();
  for (int o = 1; o < kPermuteThreads; o <<= 1) {  // Hillis-Steele inclusive scan
    const int v = threadIdx.x >= o ? scan[threadIdx.x - o] : 0;
    __syncthreads();
    scan[threadIdx.x] += v;
    __syncthreads();
  }
  int run = scan[threadIdx.x] - local;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x * 4 + q;
    if (e < E) {
      off[e] = run;
      offsets[e] = run;
    }
    run += kept4[q];
  }
  const int n_kept = scan[kPermuteThreads - 1];
  if (threadIdx.x == 0) {
    off[E] = n_kept;
    offsets[E] = n_kept;
  }
  for (int64_t p = n_kept + threadIdx.x; p < max_kept; p += kPermuteThreads) sorted_slot[p] = -1;
  __syncthreads();
  rank_and_write(ex, wbase + wave * E, s_wave, ebits, capacity, off, sorted_slot, pos, drop);
}

}  // namespace
}  // namespace moe

#endif  // MOE_PERMUTE_BLOCK_H_

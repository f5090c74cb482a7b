// Device pieces of the router shared by the router launches (router.hip) and the decode
// launch that routes a single token itself (grouped_mlp_small.hip): the 64-bit selection key
// and its wave maximum, the block router for small expert counts, and the one-wave permute.
// Pages: shubhamtatvamasi.com/llm-inference/moe "Mixture of Experts", section "The router" and
// Q&A "How does a top-k router work?" (scores, top-k, gates renormalised over the chosen k);
// klaylearn.com/glossary/mixture-of-experts (tokens permuted by destination expert).
#pragma once

#include "common.h"

namespace moe {
namespace {

// Selection key of expert e with logit v: one unsigned 64-bit compare orders candidates by
// larger logit, then lower index (the selection rule). High word: the logit's bits mapped so
// that unsigned order is float order (-0 taken as +0, so the zeros tie; NaN below -inf, so it
// is chosen last); low word: 0x7FFFFFFF - e. Keys are distinct for distinct experts.
__device__ __forceinline__ uint64_t select_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  o = (u & 0x7FFFFFFFu) > 0x7F800000u ? 0u : o;
  return (static_cast<uint64_t>(o) << 32) | static_cast<uint32_t>(0x7FFFFFFF - e);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return 0x7FFFFFFF - static_cast<int>(static_cast<uint32_t>(key)); }
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t o = static_cast<uint32_t>(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int CTRL>
__device__ __forceinline__ void dpp_max_key_step(uint64_t& v) {
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, 0xF, 0xF, false));
  const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
  v = o > v ? o : v;
}

// Row (16-lane) maximum of a key: lane ^ 1, lane ^ 2 (quad permutes), then the half-row and
// row mirrors, which pair every lane with one across the halves already reduced; afterwards
// every lane of the row holds the row's maximum.
__device__ __forceinline__ uint64_t row_max_key(uint64_t v) {
  dpp_max_key_step<0xB1>(v);
  dpp_max_key_step<0x4E>(v);
  dpp_max_key_step<0x141>(v);
  dpp_max_key_step<0x140>(v);
  return v;
}

__device__ __forceinline__ uint64_t read_key_lane(uint64_t v, int l) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), l));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Wave maximum of a key, returned wave-uniform: the row maxima, then the four row winners
// (lanes 0, 16, 32, 48) compared after readlane. DPP moves cost a VALU cycle; a cross-lane
// shuffle through the LDS unit about a hundred.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  v = row_max_key(v);
  uint64_t b = read_key_lane(v, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const uint64_t o = read_key_lane(v, 16 * r);
    b = o > b ? o : b;
  }
  return b;
}

// Small expert counts (E <= 32): a block of 256 threads owns TB tokens and splits d over all
// its lanes (8 consecutive elements per lane per pass), so even one token keeps 256 lanes'
// loads in flight. Every load is issued unconditionally (rows past the end are clamped to
// the last one and ignored), which keeps the compiler's count of loads in flight exact.
// Partial sums (TB * EMAX = 32 per lane) are summed through LDS in a fixed order: each
// thread folds one value over 32 lanes, then each logit over the 8 groups of lanes; wave w
// then runs top-k and the gates for token w. WIDE: blocks of more than 256 threads (a decode
// launch that routes its token itself), whose extra waves pass the same barriers idle;
// write_out = false keeps idx, gate and logits in the block (sidx only).
template <typename T, int EMAX, int TB, bool WIDE = false>
__device__ __forceinline__ void router_small_e_block(
    const T* __restrict__ x, const T* __restrict__ w, const float* __restrict__ bias,
    int32_t* __restrict__ idx, float* __restrict__ gate, float* __restrict__ logits, int n_tok,
    int d, int E, int k, int gating, int blk, int* sidx = nullptr, bool write_out = true) {
  static_assert(TB * EMAX == 32, "32 partial sums per lane");
  __shared__ float part[256][33];  // +1: rows fall on distinct banks
  __shared__ float red[8][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blk * TB;
  float acc[TB * EMAX];
#pragma unroll
  for (int i = 0; i < TB * EMAX; ++i) acc[i] = 0.f;
  const T* xr[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) xr[b] = x + static_cast<int64_t>(min(t0 + b, n_tok - 1)) * d;
  const T* wr[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) wr[e] = w + static_cast<int64_t>(min(e, E - 1)) * d;
  // raw 16-byte vectors (bf16: 8 values, fp32: two of them) are kept until the multiply, so
  // the loads of a pass need few registers
  constexpr int kVec = sizeof(T) == 2 ? 1 : 2;
  auto widen = [](const u32x4 (&r)[kVec], float (&v)[8]) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(r[0][i] << 16);
        v[2 * i + 1] = __uint_as_float(r[0][i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(r[i / 4][i % 4]);
    }
  };
  // d is a multiple of 64, so a lane's 8 elements never straddle the end. With few rows per
  // pass (E <= 8, bf16), two passes of the block (4096 elements) are loaded before either is
  // multiplied: at decode batch sizes the block's time is the latency of its load rounds.
  constexpr int NP = (TB + EMAX) * kVec <= 12 ? 2 : 1;
  auto fma_pass = [&](const u32x4 (&xraw)[TB][kVec], const u32x4 (&wraw)[EMAX][kVec]) {
    float xv[TB][8];
#pragma unroll
    for (int b = 0; b < TB; ++b) widen(xraw[b], xv[b]);
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      float wv[8];
      widen(wraw[e], wv);
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[b * EMAX + e] = fmaf(xv[b][i], wv[i], acc[b * EMAX + e]);
    }
  };
  const bool member = !WIDE || threadIdx.x < 256;  // wave-uniform
  for (int c = threadIdx.x * 8; member && c < d; c += NP * 2048) {
    u32x4 xr_raw[NP][TB][kVec], wr_raw[NP][EMAX][kVec];
#pragma unroll
    for (int h = 0; h < NP; ++h) {
      const int ch = c + h * 2048;
      if (ch >= d) break;
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int q = 0; q < kVec; ++q) xr_raw[h][b][q] = *reinterpret_cast<const u32x4*>(xr[b] + ch + 4 * q);
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
#pragma unroll
        for (int q = 0; q < kVec; ++q) wr_raw[h][e][q] = *reinterpret_cast<const u32x4*>(wr[e] + ch + 4 * q);
    }
#pragma unroll
    for (int h = 0; h < NP; ++h)
      if (c + h * 2048 < d) fma_pass(xr_raw[h], wr_raw[h]);
  }
  if (member) {
#pragma unroll
    for (int i = 0; i < 32; ++i) part[threadIdx.x][i] = acc[i];
  }
  __syncthreads();
  if (member) {
    const int o = threadIdx.x & 31, grp = threadIdx.x >> 5;
    float sum = 0.f;
    for (int l = 0; l < 32; ++l) sum += part[grp * 32 + l][o];
    red[grp][o] = sum;
  }
  __syncthreads();
  const int t = t0 + wave;
  if (wave >= TB || t >= n_tok) return;  // (the caller's block continues past this function)
  float my = -INFINITY;
  if (lane < E) {
    const int j = wave * EMAX + lane;
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) sum += red[g][j];
    my = sum + (bias ? bias[lane] : 0.f);
  }
  if (write_out && logits && lane < E) logits[static_cast<int64_t>(t) * E + lane] = my;
  // top-k: k rounds of a wave maximum over the selection keys below the previous winner's
  const uint64_t key = lane < E ? select_key(my, lane) : 0ull;
  uint64_t last = ~0ull;
  float first = 0.f, mine_l = 0.f;
  int mine_e = 0;
  for (int j = 0; j < k; ++j) {
    const uint64_t best = wave_max_key(key < last ? key : 0ull);
    last = best;
    const float bl = key_logit(best);
    if (lane == j) { mine_l = bl; mine_e = key_expert(best); }
    if (j == 0) first = bl;
  }
  float p = 0.f;
  if (lane < k) p = (gating == MOE_SOFTMAX) ? __expf(mine_l - first) : sigmoid_f32(mine_l);
  float sum = p;
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    if (write_out) {
      idx[static_cast<int64_t>(t) * k + lane] = mine_e;
      gate[static_cast<int64_t>(t) * k + lane] = p / sum;
    }
    if (sidx) sidx[wave * k + lane] = mine_e;  // the block's pairs, for a permute in the same block
  }
}

// Permute of at most 64 pairs (a decode batch routed by this block) by one wave: ex = the
// pairs' experts from LDS (pair s = lane). Lane e < E counts expert e's pairs, a wave prefix
// sum of the capped counts gives the offsets, and a pair's rank within its expert is the
// number of lower pairs with the same expert: the order (expert, then pair, i.e. token)
// and the drops (the highest tokens beyond the capacity) of the block permute. E <= 63.
__device__ __forceinline__ void permute_tiny_wave(const int* sidx, int n_pairs, int E, int64_t capacity,
                                                  int64_t max_kept, int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
                                                  int32_t* __restrict__ pos, uint8_t* __restrict__ drop) {
  const int lane = threadIdx.x & 63;
  int e = lane < n_pairs ? sidx[lane] : -1;
  if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) e = -1;  // outside [0, E): dropped
  int cnt = 0, rank = 0;
  for (int j = 0; j < n_pairs; ++j) {
    const int ej = __shfl(e, j);
    cnt += ej == lane;
    rank += (j < lane && ej == e) ? 1 : 0;
  }
  const int kept = lane < E ? (capacity >= 0 && cnt > capacity ? static_cast<int>(capacity) : cnt) : 0;
  int incl = kept;  // inclusive prefix over the lanes
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  const int off = incl - kept;
  const int n_kept = __shfl(incl, 63);
  if (lane < E) {
    counts[lane] = cnt;
    offsets[lane] = off;
  }
  if (lane == 0) offsets[E] = n_kept;
  const int base = __shfl(off, e < 0 ? 0 : e);
  if (lane < n_pairs) {
    if (e >= 0 && (capacity < 0 || rank < capacity)) {
      sorted_slot[base + rank] = lane;
      pos[lane] = base + rank;
      drop[lane] = 0;
    } else {
      pos[lane] = -1;
      drop[lane] = 1;
    }
  }
  for (int64_t q = n_kept + lane; q < max_kept; q += 64) sorted_slot[q] = -1;
}

}  // namespace
}  // namespace moe

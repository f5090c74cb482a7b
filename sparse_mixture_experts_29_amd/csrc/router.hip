// Router: logits = x . W_r^T + b, top-k per token (ties to the lower expert index), gates
// renormalised over the chosen k (softmax, or sigmoid as in DeepSeek-V3).
// Pages: shubhamtatvamasi.com/llm-inference/moe "Mixture of Experts", section "The router"
// and Q&A "How does a top-k router work?"; shipai.vats.cc "How routing works (intuition)".
//
// E <= 8, or E <= 32 with a small batch: vector-ALU kernel (router_small_e_kernel).
// Larger E: one block of 256 threads owns BT tokens and every expert:
//   1. logits tile [BT][E] accumulated in fp32 (bf16: MFMA 16x16x32, W_r rows as the A
//      operand, token rows as B; fp32: plain FMA) and parked in LDS;
//   2. each wave takes BT/4 tokens (E <= 256: a row of 16 lanes per token) and runs k
//      rounds of a maximum over the token's selection keys, one 64-bit key per expert that
//      orders by larger logit, then lower index; then the gates.
// Every path (also the small-E kernel) selects through the same keys.
// The bf16 K loop reads 32 contiguous bytes per lane per operand per 64-wide K block and
// feeds them to 2 MFMAs; the MFMA sees a permuted K order, identical for both operands, so
// the dot products are unchanged.
#include "common.h"
#include "route_block.h"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;
// tokens per block of the bf16 MFMA router: 32, or 64 for batches that still give every CU a
// block (every block reads all of W_r, so 64-token blocks halve those reads)
constexpr int kRouterBT = 32;
constexpr int kRouterBTLarge = 64;

// Row (16-lane) sum: after the four DPP steps every lane of a row holds the row's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_sum_step(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row_sum(float v) {
  v = dpp_sum_step<0xB1>(v);
  v = dpp_sum_step<0x4E>(v);
  v = dpp_sum_step<0x141>(v);
  return dpp_sum_step<0x140>(v);
}

// Top-k and gates for E <= 16 R: each row of 16 lanes owns one token (a wave runs 4 tokens at
// once) and lane li holds the selection keys of candidates li, li+16, ... in registers. Round
// j takes the row maximum among keys below the previous winner's (keys are distinct, so this
// walks the candidates in selection order). Slot j is kept by lane j % 16 (k <= 32).
template <int BT, int R>
__device__ void topk_rows(const float* lg, int ld, int t0, int T, int E, int k, int gating, int32_t* idx,
                          float* gate) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, rq = lane >> 4;
  constexpr int kTokPerWave = BT / 4;
  for (int tt = 0; tt < kTokPerWave; tt += 4) {
    const int tl = wave * kTokPerWave + tt + rq;
    const int t = t0 + tl;
    const bool live = tt + rq < kTokPerWave && t < T;
    const float* row = lg + (live ? tl : 0) * ld;
    uint64_t key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = li + 16 * r;
      key[r] = e < E ? select_key(row[e], e) : 0ull;  // 0: below every real key
    }
    uint64_t last = ~0ull;
    float first = 0.f, my_l[2] = {0.f, 0.f};
    int my_e[2] = {0, 0};
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) best = key[r] < last && key[r] > best ? key[r] : best;
      best = row_max_key(best);
      last = best;
      const float bl = key_logit(best);
      if (li == (j & 15)) {
        my_l[j >> 4] = bl;
        my_e[j >> 4] = key_expert(best);
      }
      if (j == 0) first = bl;
    }
    float p[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = li + 16 * h;
      p[h] = j < k ? (gating == MOE_SOFTMAX ? __expf(my_l[h] - first) : sigmoid_f32(my_l[h])) : 0.f;
    }
    const float sum = row_sum(p[0] + p[1]);
    if (live) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = li + 16 * h;
        if (j < k) {
          idx[static_cast<int64_t>(t) * k + j] = my_e[h];
          gate[static_cast<int64_t>(t) * k + j] = p[h] / sum;
        }
      }
    }
  }
}

// Top-k and gates of the tokens of a block, from their logits in LDS (row tl at lg + tl*ld).
// Each wave takes BT/4 tokens; lane l holds the selection keys of candidates l, l+64, ...
// (E <= 1024) and k rounds of a wave maximum over the keys below the previous winner's pick
// the experts in descending order.
template <int BT>
__device__ void topk_and_gates(const float* lg, int ld, int t0, int T, int E, int k, int gating,
                               int32_t* idx, float* gate) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kTokPerWave = BT / 4;
  constexpr int RMAX = 16;      // E <= 1024
  const int R = (E + 63) / 64;  // candidates per lane
  for (int tt = 0; tt < kTokPerWave; ++tt) {
    const int tl = wave * kTokPerWave + tt;
    const int t = t0 + tl;
    if (t >= T) break;
    const float* row = lg + tl * ld;
    uint64_t key[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      const int e = lane + 64 * r;
      key[r] = (r < R && e < E) ? select_key(row[e], e) : 0ull;
    }
    uint64_t last = ~0ull;
    float first = 0.f, my_l = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int r = 0; r < RMAX; ++r) best = key[r] < last && key[r] > best ? key[r] : best;
      best = wave_max_key(best);
      last = best;
      const float bl = key_logit(best);
      if (lane == j) {
        my_l = bl;
        my_e = key_expert(best);
      }
      if (j == 0) first = bl;
    }
    // gates over the k chosen logits held by lanes 0..k-1
    float p = 0.f;
    if (lane < k) p = (gating == MOE_SOFTMAX) ? __expf(my_l - first) : sigmoid_f32(my_l);
    float sum = p;
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane < k) {
      idx[static_cast<int64_t>(t) * k + lane] = my_e;
      gate[static_cast<int64_t>(t) * k + lane] = p / sum;
    }
  }
}

// Top-k and gates from a block's logits in LDS: E <= 256 by rows of 16 lanes with as few
// candidates per lane as E needs, larger E by whole waves.
template <int BT>
__device__ __forceinline__ void topk_block(const float* lg, int ld, int t0, int T, int E, int k, int gating,
                                           int32_t* idx, float* gate) {
  if (E <= 64)
    topk_rows<BT, 4>(lg, ld, t0, T, E, k, gating, idx, gate);
  else if (E <= 128)
    topk_rows<BT, 8>(lg, ld, t0, T, E, k, gating, idx, gate);
  else if (E <= 256)
    topk_rows<BT, 16>(lg, ld, t0, T, E, k, gating, idx, gate);
  else
    topk_and_gates<BT>(lg, ld, t0, T, E, k, gating, idx, gate);
}

// One pass of the bf16 router for one wave: NJ expert tiles of 16 (tiles p0 + wave + 4j) x
// NT token tiles of 16, logits (+ bias) parked in LDS. K is read in blocks of 64: lane
// (row l16, quad) holds k in [kb + 16*quad, +16) as two 16-byte loads (the same permuted
// order for both operands), through a ring of 3 register sets: block i+2 is loaded while
// block i is multiplied. d is a multiple of 64, so there is no K tail.
template <int NJ, int NT>
__device__ __forceinline__ void router_pass(const bf16_t* __restrict__ w, const bf16_t* const (&xrow)[NT],
                                            const float* __restrict__ bias, float* lg, int ld, int d, int E,
                                            int p0, int wave, int quad, int l16) {
  const int nkb = d / 64;
  const bf16_t* wrow[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    int e = (p0 + wave + 4 * j) * 16 + l16;
    e = e < E ? e : E - 1;
    wrow[j] = w + static_cast<int64_t>(e) * d;
  }
  f32x4 acc[NJ][NT];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[j][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  struct Ops {
    u32x4 a[NJ][2], b[NT][2];
  };
  auto load = [&](Ops& o, int blk) {
    const int ko = blk * 64 + quad * 16;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) o.a[j][c] = *reinterpret_cast<const u32x4*>(wrow[j] + ko + c * 8);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o.b[nt][c] = *reinterpret_cast<const u32x4*>(xrow[nt] + ko + c * 8);
    }
  };
  auto mma = [&](const Ops& o) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[j][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, o.a[j][c]),
                                                               __builtin_bit_cast(bf16x8, o.b[nt][c]),
                                                               acc[j][nt], 0, 0, 0);
  };
  constexpr int D = 3;
  Ops o[D];
#pragma unroll
  for (int j = 0; j < D - 1; ++j) load(o[j], min(j, nkb - 1));
  int i = 0;
  for (; i + 2 * D - 1 <= nkb; i += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      load(o[(j + D - 1) % D], i + j + D - 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(o[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int j = 0; j < D; ++j) {
    if (i + j + D - 1 < nkb) load(o[(j + D - 1) % D], i + j + D - 1);
    if (i + j < nkb) mma(o[j]);
  }
#pragma unroll
  for (int j = 0; j < D - 1; ++j)
    if (i + D + j < nkb) mma(o[j]);
  // C layout (16x16): lane holds rows (experts) 4*quad + r of its tile, column (token) l16
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = (p0 + wave + 4 * j) * 16 + quad * 4 + r;
        if (e < E) lg[(nt * 16 + l16) * ld + e] = acc[j][nt][r] + (bias ? bias[e] : 0.f);
      }
}

template <int BT>
__global__ __launch_bounds__(kRouterThreads) void router_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, const float* __restrict__ bias,
    int32_t* __restrict__ idx, float* __restrict__ gate, float* __restrict__ logits, int T, int d,
    int E, int k, int gating) {
  extern __shared__ float lg[];  // [BT][ld]
  const int ld = E + 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * BT;
  constexpr int NT = BT / 16;  // token tiles of 16
  const int quad = lane >> 4, l16 = lane & 15;

  // token rows this lane reads (clamped; rows past T are computed and discarded)
  const bf16_t* xrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int t = t0 + nt * 16 + l16;
    t = t < T ? t : T - 1;
    xrow[nt] = x + static_cast<int64_t>(t) * d;
  }

  // Expert tiles of 16 go round-robin to the waves, at most 4 per wave per pass of 256
  // experts, so all 4 waves work for any E >= 64; a wave runs the pass with exactly its
  // number of live tiles (1..4).
  const int n_et = (E + 15) / 16;
  for (int p0 = 0; p0 < n_et; p0 += 16) {
    const int nj = __builtin_amdgcn_readfirstlane(min(4, max(0, (n_et - p0 - wave + 3) / 4)));
    if (nj == 4)
      router_pass<4, NT>(w, xrow, bias, lg, ld, d, E, p0, wave, quad, l16);
    else if (nj == 3)
      router_pass<3, NT>(w, xrow, bias, lg, ld, d, E, p0, wave, quad, l16);
    else if (nj == 2)
      router_pass<2, NT>(w, xrow, bias, lg, ld, d, E, p0, wave, quad, l16);
    else if (nj == 1)
      router_pass<1, NT>(w, xrow, bias, lg, ld, d, E, p0, wave, quad, l16);
  }
  __syncthreads();
  if (logits) {
    for (int i = threadIdx.x; i < BT * E; i += kRouterThreads) {
      const int tl = i / E, e = i - tl * E;
      if (t0 + tl < T) logits[static_cast<int64_t>(t0 + tl) * E + e] = lg[tl * ld + e];
    }
  }
  topk_block<BT>(lg, ld, t0, T, E, k, gating, idx, gate);
}

// ---------------------------------------------------------------- LDS-staged logits (bf16)
// E <= 256: the logits tile [BT][E] of a block from operands staged through LDS by
// direct-to-LDS loads. A direct operand load of the 16x16x32 MFMA touches 16 rows, 16 cache
// lines, per instruction, and a loop built on such loads ran at the rate of its load
// instructions (dropping either operand's loads halved it); a DMA instruction fills 8 whole
// 128-byte rows (1 KB). A stage holds EW rows of W_r (E rounded up to a multiple of 64; rows
// past E repeat row E-1 and their logits are dropped), then the BT token rows (past T: row
// T-1), 64 k (128 bytes) per row; 16-byte chunk slot p of row r holds the row's chunk
// p ^ (r & 7), so the 16 rows of an operand read spread over the banks. The ring holds as
// many stages as fit about 120 KB (3..8): with little MFMA work per stage, its bytes in
// flight are what hide the load latency.
__host__ __device__ constexpr int router_lds_rows(int BT, int EW) { return EW + BT; }
__host__ __device__ constexpr int router_lds_nst(int BT, int EW) {
  return 122880 / (router_lds_rows(BT, EW) * 128) > 8   ? 8
         : 122880 / (router_lds_rows(BT, EW) * 128) < 3 ? 3
                                                         : 122880 / (router_lds_rows(BT, EW) * 128);
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left at their maximum (gfx9 encoding)
template <int N>
__device__ __forceinline__ void router_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// this wave's DMA of the current stage has landed once at most `later` later stages (IPW
// instructions each) are still in flight
template <int IPW, int NST>
__device__ __forceinline__ void router_wait_stage(int later) {
  static_assert(NST <= 8 && (NST - 2) * IPW < 64, "the wait counter holds the stages in flight");
  switch (later) {
    case 0: router_wait_vmcnt<0>(); break;
    case 1: router_wait_vmcnt<IPW>(); break;
    case 2: router_wait_vmcnt<(NST > 3 ? 2 : 1) * IPW>(); break;
    case 3: router_wait_vmcnt<(NST > 4 ? 3 : 1) * IPW>(); break;
    case 4: router_wait_vmcnt<(NST > 5 ? 4 : 1) * IPW>(); break;
    case 5: router_wait_vmcnt<(NST > 6 ? 5 : 1) * IPW>(); break;
    default: router_wait_vmcnt<(NST > 7 ? 6 : 1) * IPW>(); break;
  }
}

// bare workgroup barrier: every wave has already waited for its own DMA (__syncthreads
// would also drain the DMA still in flight); the empty asm keeps memory accesses in place
__device__ __forceinline__ void router_stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct-to-LDS 16-byte load: lane l's 16 bytes at g land at LDS byte address m0 + 16 l. No
// register result; M0 is written here and declared clobbered, one wait state before use.
// The loop orders it with its own vmcnt waits and barriers.
__device__ __forceinline__ void router_dma16(const char* g, uint32_t lds_byte) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(m0v) : "memory", "m0");
}

typedef __attribute__((address_space(3))) void router_lds_void;

template <int BT, int EW>
__global__ __launch_bounds__(kRouterThreads) void router_bf16_lds_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, const float* __restrict__ bias,
    int32_t* __restrict__ idx, float* __restrict__ gate, float* __restrict__ logits, int T, int d,
    int E, int k, int gating) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];  // the stage ring, then the logits
  constexpr int ROWS = router_lds_rows(BT, EW);
  constexpr int STAGE = ROWS * 128;  // bytes
  constexpr int IPW = ROWS / 32;     // DMA instructions per wave per stage (8 rows each)
  constexpr int NST = router_lds_nst(BT, EW);
  constexpr int NJ = EW / 64;  // expert tiles of 16 per wave (tiles wave, wave + 4, ...)
  constexpr int NT = BT / 16;  // token tiles of 16
  static_assert(ROWS % 32 == 0 && EW % 64 == 0, "whole DMA instructions per wave");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int quad = lane >> 4, l16 = lane & 15;
  const int t0 = blockIdx.x * BT;
  const int nkb = d / 64;

  // instruction i of this wave fills stage rows 8 q .. 8 q + 7, q = 4 i + wave; lane l takes
  // row 8 q + l / 8 and stores its chunk slot l % 8 = logical chunk (l % 8) ^ (row & 7)
  const char* src[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = 8 * (4 * i + wave) + (lane >> 3);
    const int p = (lane & 7) ^ (r & 7);
    const bf16_t* row = r < EW ? w + static_cast<int64_t>(min(r, E - 1)) * d
                               : x + static_cast<int64_t>(min(t0 + r - EW, T - 1)) * d;
    src[i] = reinterpret_cast<const char*>(row) + p * 16;
  }
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((router_lds_void*)smem));
  auto issue = [&](int kb) {
    const uint32_t st = lds0 + static_cast<uint32_t>((kb % NST) * STAGE);
#pragma unroll
    for (int i = 0; i < IPW; ++i) router_dma16(src[i] + static_cast<int64_t>(kb) * 128, st + (4 * i + wave) * 1024);
  };
  // operand byte offsets within a stage, k half c: row r, logical chunk 4 c + quad
  int aoff[NJ][2], boff[NT][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = 16 * (wave + 4 * j) + l16;
      aoff[j][c] = r * 128 + (((4 * c + quad) ^ (r & 7)) * 16);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = EW + 16 * nt + l16;
      boff[nt][c] = r * 128 + (((4 * c + quad) ^ (r & 7)) * 16);
    }
  }

  f32x4 acc[NJ][NT];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[j][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nkb) issue(s);
  for (int kb = 0; kb < nkb; ++kb) {
    router_wait_stage<IPW, NST>(min(NST - 2, nkb - 1 - kb));
    router_stage_barrier();  // stage kb is complete; every wave is done with stage kb - 1's slot
    if (kb + NST - 1 < nkb) issue(kb + NST - 1);
    const char* st = smem + (kb % NST) * STAGE;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 a[NJ], b[NT];
#pragma unroll
      for (int j = 0; j < NJ; ++j) a[j] = *reinterpret_cast<const u32x4*>(st + aoff[j][c]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) b[nt] = *reinterpret_cast<const u32x4*>(st + boff[nt][c]);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[j][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[j]),
                                                               __builtin_bit_cast(bf16x8, b[nt]), acc[j][nt], 0, 0, 0);
    }
  }
  router_stage_barrier();  // every wave is done reading the ring; the logits tile reuses it
  float* lg = reinterpret_cast<float*>(smem);
  const int ld = E + 4;
  // C layout (16x16): lane holds rows (experts) 4 quad + r of its tile, column (token) l16
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 16 * (wave + 4 * j) + quad * 4 + r;
        if (e < E) lg[(nt * 16 + l16) * ld + e] = acc[j][nt][r] + (bias ? bias[e] : 0.f);
      }
  __syncthreads();
  if (logits) {
    for (int i = threadIdx.x; i < BT * E; i += kRouterThreads) {
      const int tl = i / E, e = i - tl * E;
      if (t0 + tl < T) logits[static_cast<int64_t>(t0 + tl) * E + e] = lg[tl * ld + e];
    }
  }
  topk_block<BT>(lg, ld, t0, T, E, k, gating, idx, gate);
}

template <int BT>
__global__ __launch_bounds__(kRouterThreads) void router_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    int32_t* __restrict__ idx, float* __restrict__ gate, float* __restrict__ logits, int T, int d,
    int E, int k, int gating) {
  extern __shared__ float lg[];
  const int ld = E + 4;
  const int t0 = blockIdx.x * BT;
  for (int i = threadIdx.x; i < BT * E; i += kRouterThreads) {
    const int tl = i / E, e = i - tl * E;
    const int t = t0 + tl < T ? t0 + tl : T - 1;
    const float* xr = x + static_cast<int64_t>(t) * d;
    const float* wr = w + static_cast<int64_t>(e) * d;
    float s = 0.f;
    for (int c = 0; c < d; c += 4) {
      const float4 xv = *reinterpret_cast<const float4*>(xr + c);
      const float4 wv = *reinterpret_cast<const float4*>(wr + c);
      s = fmaf(xv.x, wv.x, s);
      s = fmaf(xv.y, wv.y, s);
      s = fmaf(xv.z, wv.z, s);
      s = fmaf(xv.w, wv.w, s);
    }
    lg[tl * ld + e] = s + (bias ? bias[e] : 0.f);
  }
  __syncthreads();
  if (logits) {
    for (int i = threadIdx.x; i < BT * E; i += kRouterThreads) {
      const int tl = i / E, e = i - tl * E;
      if (t0 + tl < T) logits[static_cast<int64_t>(t0 + tl) * E + e] = lg[tl * ld + e];
    }
  }
  topk_block<BT>(lg, ld, t0, T, E, k, gating, idx, gate);
}

template <typename T, int EMAX, int TB>
__global__ __launch_bounds__(256) void router_small_e_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const float* __restrict__ bias,
    int32_t* __restrict__ idx, float* __restrict__ gate, float* __restrict__ logits, int n_tok,
    int d, int E, int k, int gating) {
  router_small_e_block<T, EMAX, TB>(x, w, bias, idx, gate, logits, n_tok, d, E, k, gating, blockIdx.x);
}

// Route and permute in one launch when both fit one block (the router's single block of TB
// tokens, at most 32 pairs): the block's top-k choices are also kept in LDS, and after a
// barrier one wave permutes them (permute_tiny_wave). Saves a launch and its gap on decode
// steps, and the one-block permute's scan and its global round trip of the choices (about
// 2 us a step, measured at T = 1 and 4); the results are those of the two separate launches.
template <typename T, int EMAX, int TB>
__global__ __launch_bounds__(256) void route_permute_single_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const float* __restrict__ bias,
    int32_t* __restrict__ idx, float* __restrict__ gate, float* __restrict__ logits, int n_tok,
    int d, int E, int k, int gating, int64_t capacity, int64_t max_kept,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ pos, uint8_t* __restrict__ drop) {
  // the pairs (at most TB * k <= 32) stay in LDS; one wave permutes them
  __shared__ int sidx[64];
  router_small_e_block<T, EMAX, TB>(x, w, bias, idx, gate, logits, n_tok, d, E, k, gating, 0, sidx);
  __syncthreads();
  if (threadIdx.x < 64)
    permute_tiny_wave(sidx, n_tok * k, E, capacity, max_kept, counts, offsets, sorted_slot, pos, drop);
}
}  // namespace

hipError_t launch_route(const Shape& s, const void* x, const void* w_router, const float* bias,
                        int32_t* idx, float* gate, float* logits, hipStream_t st) {
  const int T = static_cast<int>(s.T);
  // up to 8 experts: 4 tokens per block; up to 32: 1 token per block, for small batches only
  // (every block reads all of W_r; the MFMA kernel below reads it once per 64 tokens)
  if (s.E <= 8 || (s.E <= 32 && T <= 256)) {
    const bool e8 = s.E <= 8;
    const dim3 g(e8 ? (T + 3) / 4 : T), b(kRouterThreads);
    timing_begin(MOE_KERNEL_ROUTER, st);
    if (s.dtype == MOE_BF16) {
      auto kern = e8 ? router_small_e_kernel<bf16_t, 8, 4> : router_small_e_kernel<bf16_t, 32, 1>;
      hipLaunchKernelGGL(kern, g, b, 0, st, static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w_router),
                         bias, idx, gate, logits, T, s.d, s.E, s.k, s.gating);
    } else {
      auto kern = e8 ? router_small_e_kernel<float, 8, 4> : router_small_e_kernel<float, 32, 1>;
      hipLaunchKernelGGL(kern, g, b, 0, st, static_cast<const float*>(x), static_cast<const float*>(w_router),
                         bias, idx, gate, logits, T, s.d, s.E, s.k, s.gating);
    }
    timing_end(MOE_KERNEL_ROUTER, st);
    return hipGetLastError();
  }
  const dim3 block(kRouterThreads);
  timing_begin(MOE_KERNEL_ROUTER, st);
  if (s.dtype == MOE_BF16) {
    // 32 tokens per block, or 64 once T gives every CU a 64-token block and E <= 256: every
    // block reads all of W_r, so larger blocks read it fewer times, while below that T the
    // idle CUs cost more (measured on the direct-load kernel: DeepSeek-shaped, T = 16384,
    // E = 256, d = 7168: 335 -> 236 us with 64; qwen3_fine, T = 8192: 48 -> 79 us). The
    // logits tile of E = 1024 still fits LDS at 32 tokens (32 x 1028 x 4 B).
    const bool large = s.E <= 256 && T / kRouterBTLarge >= cu_count();
    const int BT = large ? kRouterBTLarge : kRouterBT;
    const size_t lg_bytes = static_cast<size_t>(BT) * (s.E + 4) * sizeof(float);
    if (s.E <= 256) {
      // operands through LDS; the ring (then the logits tile) is one dynamic LDS array
      const int EW = s.E <= 64 ? 64 : (s.E <= 128 ? 128 : 256);
      const size_t ring = static_cast<size_t>(router_lds_nst(BT, EW)) * router_lds_rows(BT, EW) * 128;
      const size_t lds = std::max(ring, lg_bytes);
      auto kern = large ? (EW == 64 ? router_bf16_lds_kernel<kRouterBTLarge, 64>
                                    : EW == 128 ? router_bf16_lds_kernel<kRouterBTLarge, 128>
                                                : router_bf16_lds_kernel<kRouterBTLarge, 256>)
                        : (EW == 64 ? router_bf16_lds_kernel<kRouterBT, 64>
                                    : EW == 128 ? router_bf16_lds_kernel<kRouterBT, 128>
                                                : router_bf16_lds_kernel<kRouterBT, 256>);
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                static_cast<int>(lds));
      hipLaunchKernelGGL(kern, dim3((T + BT - 1) / BT), block, lds, st, static_cast<const bf16_t*>(x),
                         static_cast<const bf16_t*>(w_router), bias, idx, gate, logits, T, s.d, s.E,
                         s.k, s.gating);
    } else {
      auto kern = router_bf16_kernel<kRouterBT>;
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                static_cast<int>(lg_bytes));
      hipLaunchKernelGGL(kern, dim3((T + kRouterBT - 1) / kRouterBT), block, lg_bytes, st,
                         static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w_router), bias, idx, gate,
                         logits, T, s.d, s.E, s.k, s.gating);
    }
  } else {
    const bool small_e = s.E <= 256;
    const int BT = small_e ? 64 : 16;
    const size_t lds = static_cast<size_t>(BT) * (s.E + 4) * sizeof(float);
    auto kern = small_e ? router_f32_kernel<64> : router_f32_kernel<16>;
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(lds));
    hipLaunchKernelGGL(kern, dim3((T + BT - 1) / BT), block, lds, st, static_cast<const float*>(x),
                       static_cast<const float*>(w_router), bias, idx, gate, logits, T, s.d, s.E,
                       s.k, s.gating);
  }
  timing_end(MOE_KERNEL_ROUTER, st);
  return hipGetLastError();
}

hipError_t launch_route_permute(const Shape& s, const void* x, const void* w_router, const float* bias,
                                int32_t* idx, float* gate, float* logits, int32_t* counts, int32_t* offsets,
                                int32_t* sorted_slot, int32_t* pos, uint8_t* drop, void* permute_ws,
                                hipStream_t st) {
  const int T = static_cast<int>(s.T);
  // one router block (E <= 8: 4 tokens; E <= 32: 1 token) and one permute chunk
  const bool e8 = s.E <= 8;
  const bool one_block = (e8 && T <= 4) || (s.E <= 32 && T == 1);
  if (!one_block || s.T * s.k > kPermuteChunk) {
    hipError_t e = launch_route(s, x, w_router, bias, idx, gate, logits, st);
    if (e == hipSuccess) e = launch_permute(s, idx, counts, offsets, sorted_slot, pos, drop, permute_ws, st);
    return e;
  }
  timing_begin(MOE_KERNEL_ROUTER, st);
  const dim3 g(1), b(kRouterThreads);
  if (s.dtype == MOE_BF16) {
    auto kern = e8 ? route_permute_single_kernel<bf16_t, 8, 4> : route_permute_single_kernel<bf16_t, 32, 1>;
    hipLaunchKernelGGL(kern, g, b, 0, st, static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w_router), bias,
                       idx, gate, logits, T, s.d, s.E, s.k, s.gating, s.capacity, s.max_kept, counts, offsets,
                       sorted_slot, pos, drop);
  } else {
    auto kern = e8 ? route_permute_single_kernel<float, 8, 4> : route_permute_single_kernel<float, 32, 1>;
    hipLaunchKernelGGL(kern, g, b, 0, st, static_cast<const float*>(x), static_cast<const float*>(w_router), bias,
                       idx, gate, logits, T, s.d, s.E, s.k, s.gating, s.capacity, s.max_kept, counts, offsets,
                       sorted_slot, pos, drop);
  }
  timing_end(MOE_KERNEL_ROUTER, st);
  return hipGetLastError();
}

}  // namespace moe

// Grouped expert MLP for small batches (decode): every group holds at most 64 rows, so
// the weights dominate the traffic and each weight element must be read from HBM once.
// Pages: shubhamtatvamasi.com/llm-inference/moe, "Memory vs compute, quantified" and the Q&A
// on batch size and decode (at small batches only the touched experts' weights are read,
// and each step streams them from memory); klaylearn.com/glossary/mixture-of-experts
// (decode gives tiny expert batches).
//
// One wave owns 16 weight rows (16 output columns) of one group and streams them straight
// from HBM into the A operand of v_mfma_f32_16x16x32_bf16: lane l holds row l%16 and the 32
// k values [32*(l/16), 32*(l/16)+32) of each 128-wide K block, as four 16-byte loads. The
// token rows (operand B, one or two groups of 16 per wave) are read with the same K order,
// so the MFMA sees a permuted K identical for both operands and the dot products are
// unchanged. Operands (weights and token rows) are loaded two K blocks ahead through a ring of three
// register sets.
//   gated launch: h = silu(v Wg) * (v Wu) for 16 columns of f, all rows of the group; when
//                 K is split, fp32 partials of both products, and a second kernel sums
//                 them in split order and applies silu * mul;
//   down launch:  split-K partial sums of h Wd in fp32, reduced in a fixed order by a
//                 second kernel (deterministic, no atomics).
// Work units = (token half, group, K split, 16-column chunk); units of empty groups exit at
// once. K splits keep the units small, so the last, partly filled round of waves is short.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;  // 4 waves, one unit each

struct SmallArgs {
  const bf16_t* in_r;          // routed input rows: x [T][K] (gather) or h [max_kept][K]
  const bf16_t* in_s;          // shared input rows: x [T][K] or hs [n_s*T][K]
  const int32_t* sorted_slot;  // gated launch: routed rows gather x[sorted_slot[p] / k]
  const int32_t* offsets;      // [E+1]
  const void* w0_r;            // [E][N_r][K_r] bf16, or FP8 E4M3 codes (one byte each)
  const void* w1_r;
  const void* w0_s;            // [n_s][N_s][K_s]
  const void* w1_s;
  const float* s0_r;           // FP8 weights: per-output-row scales [E][N_r] (else null)
  const float* s1_r;
  const float* s0_s;           // FP8 weights: shared experts' scales [n_s][N_s]
  const float* s1_s;
  bf16_t* out_r;               // gated: h [max_kept][N_r]
  bf16_t* out_s;               // gated: hs [n_s*T][N_s]
  float* part;                 // K-split partials: gated [splits][rows][2][fw], down [splits][rows][N]
  int N_r, K_r, N_s, K_s;
  int E, k, T, n_shared;
  int n_chunks;                // 16-column chunks of the widest group
  int splits;                  // K splits; gated with 1 split writes h directly
  int halves;                  // waves per (group, split, chunk), each NGW token groups
  int fw;                      // gated partials: row stride is 2*fw (fw = widest N)
  int64_t max_kept;
};

// Ring depths (DW, DX) of the K loop per launch kind: gated (G) or down (D), bf16 (B) or
// FP8 (F) weights, NG token groups. The weights of block i+DW-1 and the token rows of block
// i+DX-1 are loaded while block i is multiplied. DX divides DW. Measured on the Mixtral-shaped
// decode layer (T = 1..64, bf16 and FP8): equal depths, 3 (5 for one FP8 token group), are
// the fastest; a shorter token-row lead with a deeper weight ring (4/2, 6/2, 6/3, 8/2, 8/4)
// was equal or slower everywhere.
#ifndef MOE_SM_GB1
#define MOE_SM_GB1 3, 3
#endif
#ifndef MOE_SM_GB2
#define MOE_SM_GB2 3, 3
#endif
#ifndef MOE_SM_DB1
#define MOE_SM_DB1 3, 3
#endif
#ifndef MOE_SM_DB2
#define MOE_SM_DB2 3, 3
#endif
#ifndef MOE_SM_GF1
#define MOE_SM_GF1 5, 5
#endif
#ifndef MOE_SM_GF2
#define MOE_SM_GF2 3, 3
#endif
#ifndef MOE_SM_DF1
#define MOE_SM_DF1 5, 5
#endif
#ifndef MOE_SM_DF2
#define MOE_SM_DF2 3, 3
#endif
template <bool GATED, int NG, bool FP8>
struct RingDepth {
  static constexpr int v[2] = {MOE_SM_GB1};
};
#define MOE_SM_RING(G, N, F, DEPTHS)          \
  template <>                                 \
  struct RingDepth<G, N, F> {                 \
    static constexpr int v[2] = {DEPTHS};     \
  };
MOE_SM_RING(true, 2, false, MOE_SM_GB2)
MOE_SM_RING(false, 1, false, MOE_SM_DB1)
MOE_SM_RING(false, 2, false, MOE_SM_DB2)
MOE_SM_RING(true, 1, true, MOE_SM_GF1)
MOE_SM_RING(true, 2, true, MOE_SM_GF2)
MOE_SM_RING(false, 1, true, MOE_SM_DF1)
MOE_SM_RING(false, 2, true, MOE_SM_DF2)
#undef MOE_SM_RING

// K loop and epilogue of one unit with NG (compile-time) token groups of 16: weights DW-1
// blocks ahead, token rows DX-1 blocks ahead of the multiply, so no load waits on the one
// issued before it.
// FP8 (E4M3) weights: a lane's 32 k values of a block are 32 bytes (two 16-byte loads) and
// are widened to bf16 exactly (every E4M3 value is a bf16 value) right before the multiply;
// the per-row scale multiplies the accumulator in the epilogue.
template <bool GATED, int NG, bool FP8>
__device__ __forceinline__ void small_m_unit(const SmallArgs& a, const void* w0, const void* w1,
                                             const bf16_t* const (&xp)[2], int t0, int kbeg, int kend,
                                             int quad, int l16, int M, int r0, int gi, bool shared,
                                             int N, int n0, int split) {
  constexpr int NW = FP8 ? 2 : 4;  // 16-byte weight loads per lane per block and matrix
  constexpr int DW = RingDepth<GATED, NG, FP8>::v[0];
  constexpr int DX = RingDepth<GATED, NG, FP8>::v[1];
  static_assert(DX >= 1 && DW >= DX && DW % DX == 0, "the token-row ring divides the weight ring");
  struct WOps {
    u32x4 wa[NW], wb[NW];
  };
  struct XOps {
    u32x4 xv[NG][4];
  };
  // A operand c of a block (k = ko + 8c .. +8), from the raw weight registers; m zeroes the
  // dead lanes of the tail block (FP8 code 0 is +0)
  auto wop = [&](const u32x4 (&w)[NW], int c, unsigned m) -> bf16x8 {
    if constexpr (!FP8) {
      return __builtin_bit_cast(bf16x8, w[c] & m);
    } else {
      const u32x4 raw = w[c >> 1] & m;
      const unsigned d0 = raw[(c & 1) * 2], d1 = raw[(c & 1) * 2 + 1];
      const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
      const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
      const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
      const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
      return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
  };
  auto wfull = [&](const u32x4 (&w)[NW], int c) -> bf16x8 {
    if constexpr (!FP8)
      return __builtin_bit_cast(bf16x8, w[c]);
    else
      return wop(w, c, 0xFFFFFFFFu);
  };
  f32x4 acc0[NG], acc1[NG];
#pragma unroll
  for (int t = 0; t < NG; ++t) {
    acc0[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // lane covers k in [ko, ko+32) of a 128-wide block at kb: ko = kb + 32*quad, 64 contiguous
  // bytes per lane over the block's 4 loads, so every load touches both 128-byte lines of
  // each row's 256 bytes. In the 64-wide tail (`full` false) quads 2-3 read k in [kb, kb+32)
  // instead, which is in range, and the multiply zeroes what they read. Loads are issued
  // unconditionally and left untouched until their block is multiplied, so the compiler's
  // count of loads in flight stays exact and no wait drains the ring.
  auto offs = [&](int kb, bool full) { return kb + (full || quad < 2 ? quad * 32 : 0); };
  auto load_w = [&](WOps& o, int kb, bool full) {
    const int ko = offs(kb, full);
#pragma unroll
    for (int c = 0; c < NW; ++c) {
      if constexpr (FP8) {
        o.wa[c] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(w0) + ko + c * 16);
        if (GATED) o.wb[c] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(w1) + ko + c * 16);
      } else {
        o.wa[c] = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(w0) + ko + c * 8);
        if (GATED) o.wb[c] = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(w1) + ko + c * 8);
      }
    }
  };
  auto load_x = [&](XOps& o, int kb, bool full) {
    const int ko = offs(kb, full);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < NG; ++t) o.xv[t][c] = *reinterpret_cast<const u32x4*>(xp[t] + ko + c * 8);
  };
  // m: all ones, or zero for the dead lanes of the tail block
  auto mma = [&](const WOps& w, const XOps& o, unsigned m) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < NG; ++t) {
        const bf16x8 x = __builtin_bit_cast(bf16x8, o.xv[t][c] & m);
        acc0[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop(w.wa, c, m), x, acc0[t], 0, 0, 0);
        if (GATED) acc1[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop(w.wb, c, m), x, acc1[t], 0, 0, 0);
      }
  };
  auto mma_full = [&](const WOps& w, const XOps& o) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < NG; ++t) {
        const bf16x8 x = __builtin_bit_cast(bf16x8, o.xv[t][c]);
        acc0[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfull(w.wa, c), x, acc0[t], 0, 0, 0);
        if (GATED) acc1[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfull(w.wb, c), x, acc1[t], 0, 0, 0);
      }
  };
  const int nfull = (kend - kbeg) / 128;        // full 128-wide blocks
  const bool tail = (kend - kbeg) % 128 != 0;   // then a 64-wide block
  const int nb = nfull + (tail ? 1 : 0);
  // the weights of block bw and the token rows of block bx, interleaved chunk by chunk (so
  // the registers freed by one chunk's loads are reused by the next: no spills)
  auto load_wx = [&](WOps& w, int bw, XOps& o, int bx) {
    const int kw = offs(kbeg + bw * 128, bw < nfull), kx = offs(kbeg + bx * 128, bx < nfull);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c < NW) {
        if constexpr (FP8) {
          w.wa[c] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(w0) + kw + c * 16);
          if (GATED) w.wb[c] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(w1) + kw + c * 16);
        } else {
          w.wa[c] = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(w0) + kw + c * 8);
          if (GATED) w.wb[c] = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(w1) + kw + c * 8);
        }
      }
#pragma unroll
      for (int t = 0; t < NG; ++t) o.xv[t][c] = *reinterpret_cast<const u32x4*>(xp[t] + kx + c * 8);
    }
  };
  auto load_wb = [&](WOps& o, int b) { load_w(o, kbeg + b * 128, b < nfull); };
  auto load_xb = [&](XOps& o, int b) { load_x(o, kbeg + b * 128, b < nfull); };
  auto mma_block = [&](const WOps& w, const XOps& o, int b) {
    mma(w, o, b < nfull || quad < 2 ? 0xFFFFFFFFu : 0u);
  };
  // rings: on entry to an iteration, the weights of blocks i .. i+DW-2 sit in W and the token
  // rows of blocks i .. i+DX-2 in X (block b in W[b % DW], X[b % DX]). The steady loop runs
  // while every block it loads exists (no guards inside) and never multiplies the tail block;
  // the peeled rounds after it finish the last < 2 DW - 1 blocks.
  WOps W[DW];
  XOps X[DX];
  // unconditional (a unit of fewer blocks reloads its last one): no branch ahead of the loop,
  // so the wait counts inside it stay exact
#pragma unroll
  for (int j = 0; j < DW - 1; ++j) {
    if (j < DX - 1)
      load_wx(W[j], min(j, nb - 1), X[j], min(j, nb - 1));
    else
      load_wb(W[j], min(j, nb - 1));
  }
  int i = 0;
  for (; i + 2 * DW - 1 <= nb; i += DW) {
#pragma unroll
    for (int j = 0; j < DW; ++j) {
      // issue block i+j+DW-1's weights and block i+j+DX-1's token rows before multiplying
      // block i+j; the scheduling barriers stop the compiler from hoisting the next block's
      // multiplies above these loads
      load_wx(W[(j + DW - 1) % DW], i + j + DW - 1, X[(j + DX - 1) % DX], i + j + DX - 1);
      __builtin_amdgcn_sched_barrier(0);
      mma_full(W[j], X[j % DX]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int j = 0; j < DW; ++j) {
    if (i + j + DW - 1 < nb) load_wb(W[(j + DW - 1) % DW], i + j + DW - 1);
    if (i + j + DX - 1 < nb) load_xb(X[(j + DX - 1) % DX], i + j + DX - 1);
    if (i + j < nb) mma_block(W[j], X[j % DX], i + j);
  }
#pragma unroll
  for (int j = 0; j < DW - 1; ++j) {
    if (i + DW + j + DX - 1 < nb) load_xb(X[(j + DX - 1) % DX], i + DW + j + DX - 1);
    if (i + DW + j < nb) mma_block(W[j], X[j % DX], i + DW + j);
  }

  // epilogue. 16x16 C layout: lane holds weight rows n0 + 4*quad + r (r = 0..3) for token
  // column l16 of each group.
  const int ncol = n0 + quad * 4;
  if (ncol >= N) return;
  if constexpr (FP8) {  // per-row scales of the FP8 weights
    const float* sc0 = shared ? a.s0_s : a.s0_r;
    const float* sc1 = shared ? a.s1_s : a.s1_r;
    const float4 s0 = *reinterpret_cast<const float4*>(sc0 + static_cast<int64_t>(gi) * N + ncol);
    const float4 s1 = GATED ? *reinterpret_cast<const float4*>(sc1 + static_cast<int64_t>(gi) * N + ncol) : s0;
#pragma unroll
    for (int t = 0; t < NG; ++t) {
      acc0[t] = f32x4{acc0[t][0] * s0.x, acc0[t][1] * s0.y, acc0[t][2] * s0.z, acc0[t][3] * s0.w};
      if (GATED) acc1[t] = f32x4{acc1[t][0] * s1.x, acc1[t][1] * s1.y, acc1[t][2] * s1.z, acc1[t][3] * s1.w};
    }
  }
#pragma unroll
  for (int t = 0; t < NG; ++t) {
    const int tok = (t0 + t) * 16 + l16;
    if (tok < M) {
      const int row = r0 + tok;
      if (GATED && a.splits > 1) {
        const int64_t prow = shared ? a.max_kept + static_cast<int64_t>(gi) * a.T + row : row;
        const int64_t rows_total = a.max_kept + static_cast<int64_t>(a.n_shared) * a.T;
        float* pp = a.part + (static_cast<int64_t>(split) * rows_total + prow) * 2 * a.fw + ncol;
        *reinterpret_cast<float4*>(pp) = make_float4(acc0[t][0], acc0[t][1], acc0[t][2], acc0[t][3]);
        *reinterpret_cast<float4*>(pp + a.fw) = make_float4(acc1[t][0], acc1[t][1], acc1[t][2], acc1[t][3]);
      } else if (GATED) {
        const int64_t orow = shared ? static_cast<int64_t>(gi) * a.T + row : row;
        bf16_t* op = (shared ? a.out_s : a.out_r) + orow * N + ncol;
        uint2 pk;
        pk.x = pack_bf16x2(silu_f32(acc0[t][0]) * acc1[t][0], silu_f32(acc0[t][1]) * acc1[t][1]);
        pk.y = pack_bf16x2(silu_f32(acc0[t][2]) * acc1[t][2], silu_f32(acc0[t][3]) * acc1[t][3]);
        *reinterpret_cast<uint2*>(op) = pk;
      } else {
        const int64_t prow = shared ? a.max_kept + static_cast<int64_t>(gi) * a.T + row : row;
        const int64_t rows_total = a.max_kept + static_cast<int64_t>(a.n_shared) * a.T;
        float* pp = a.part + (static_cast<int64_t>(split) * rows_total + prow) * N + ncol;
        *reinterpret_cast<float4*>(pp) = make_float4(acc0[t][0], acc0[t][1], acc0[t][2], acc0[t][3]);
      }
    }
  }
}

// NGW: token groups of 16 per wave (1 or 2, so the 3-deep ring fits the register file). A
// group with more rows than NGW*16 is covered by `halves` passes, one per NGW token groups.
// The half is the slowest unit index: in a typical small batch every group fits one half,
// and the blocks of the other halves exit at once instead of idling inside working blocks.
template <bool GATED, int NGW, bool FP8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void small_m_kernel(SmallArgs a) {
  const int lane = threadIdx.x & 63;
  // wave-uniform (readfirstlane): everything derived from the unit stays in scalar registers
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // unit = (half, group, split, chunk) with the chunk fastest: the waves of a block share a
  // group, so blocks of empty groups retire at once
  const int G = a.E + a.n_shared;
  const int nc = static_cast<int>(unit % a.n_chunks);
  int64_t rest = unit / a.n_chunks;
  const int split = static_cast<int>(rest % a.splits);
  rest /= a.splits;
  const int g = static_cast<int>(rest % G);
  const int half = static_cast<int>(rest / G);
  if (half >= a.halves) return;
  const bool shared = g >= a.E;
  const int gi = shared ? g - a.E : g;
  int r0, M;
  if (shared) {
    r0 = 0;
    M = a.T;
  } else {
    r0 = a.offsets[g];
    M = a.offsets[g + 1] - r0;
  }
  r0 = __builtin_amdgcn_readfirstlane(r0);
  M = __builtin_amdgcn_readfirstlane(M);
  const int t0 = half * NGW;            // first token group of this wave
  const int ng = ((M + 15) >> 4) - t0;  // token groups left for it
  if (ng <= 0) return;
  const int N = shared ? a.N_s : a.N_r;
  const int K = shared ? a.K_s : a.K_r;
  const int n0 = nc * 16;
  if (n0 >= N) return;
  const int ks = K / a.splits;  // multiple of 64 (host guarantees)
  const int kbeg = split * ks, kend = kbeg + ks;

  const int l16 = lane & 15, quad = lane >> 4;
  const int n = min(n0 + l16, N - 1);
  const int64_t wel = (static_cast<int64_t>(gi) * N + n) * K;  // element offset of the lane's row
  const void* w0;
  const void* w1 = nullptr;
  if constexpr (FP8) {
    w0 = static_cast<const uint8_t*>(shared ? a.w0_s : a.w0_r) + wel;
    if (GATED) w1 = static_cast<const uint8_t*>(shared ? a.w1_s : a.w1_r) + wel;
  } else {
    w0 = static_cast<const bf16_t*>(shared ? a.w0_s : a.w0_r) + wel;
    if (GATED) w1 = static_cast<const bf16_t*>(shared ? a.w1_s : a.w1_r) + wel;
  }
  const bf16_t* in = shared ? a.in_s : a.in_r;

  const bf16_t* xp[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = r0 + min((t0 + t) * 16 + l16, M - 1);
    int64_t src;
    if (shared)
      src = GATED ? r : static_cast<int64_t>(gi) * a.T + r;
    else
      src = GATED ? a.sorted_slot[r] / a.k : r;
    xp[t] = in + src * K;
  }
  if (NGW == 1 || ng <= 1)
    small_m_unit<GATED, 1, FP8>(a, w0, w1, xp, t0, kbeg, kend, quad, l16, M, r0, gi, shared, N, n0, split);
  else
    small_m_unit<GATED, 2, FP8>(a, w0, w1, xp, t0, kbeg, kend, quad, l16, M, r0, gi, shared, N, n0, split);
}

// h = silu(sum of gate partials) * (sum of up partials), the sums over K splits in split
// order, rounded once to bf16 (the gated epilogue of the K-split launch).
__global__ __launch_bounds__(256) void small_m_swiglu_reduce(const float* __restrict__ part,
                                                             const int32_t* __restrict__ offsets, int E,
                                                             int64_t max_kept, int n_shared, int T, int f,
                                                             int f_s, int fw, int splits,
                                                             bf16_t* __restrict__ h,
                                                             bf16_t* __restrict__ hs) {
  const int64_t rows_total = max_kept + static_cast<int64_t>(n_shared) * T;
  const int cq = fw / 4;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows_total * cq) return;
  const int64_t row = i / cq;
  const int c = static_cast<int>(i % cq) * 4;
  const bool routed = row < max_kept;
  if (routed ? (row >= offsets[E] || c >= f) : c >= f_s) return;
  float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
  for (int sp = 0; sp < splits; ++sp) {
    const float* pp = part + (static_cast<int64_t>(sp) * rows_total + row) * 2 * fw + c;
    const float4 vg = *reinterpret_cast<const float4*>(pp);
    const float4 vu = *reinterpret_cast<const float4*>(pp + fw);
    g.x += vg.x;
    g.y += vg.y;
    g.z += vg.z;
    g.w += vg.w;
    u.x += vu.x;
    u.y += vu.y;
    u.z += vu.z;
    u.w += vu.w;
  }
  bf16_t* op = routed ? h + row * f + c : hs + (row - max_kept) * f_s + c;
  uint2 pk;
  pk.x = pack_bf16x2(silu_f32(g.x) * u.x, silu_f32(g.y) * u.y);
  pk.y = pack_bf16x2(silu_f32(g.z) * u.z, silu_f32(g.w) * u.w);
  *reinterpret_cast<uint2*>(op) = pk;
}

// y = sum over splits of the partials, in split order, rounded once to bf16.
// One thread per 4 consecutive columns of one row; routed rows past N_kept are skipped.
__global__ __launch_bounds__(256) void small_m_reduce(const float* __restrict__ part,
                                                      const int32_t* __restrict__ offsets, int E,
                                                      int64_t max_kept, int n_shared, int T, int N,
                                                      int splits, bf16_t* __restrict__ y_perm,
                                                      bf16_t* __restrict__ y_shared) {
  const int64_t rows_total = max_kept + static_cast<int64_t>(n_shared) * T;
  const int cq = N / 4;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows_total * cq) return;
  const int64_t row = i / cq;
  const int c = static_cast<int>(i % cq) * 4;
  if (row < max_kept && row >= offsets[E]) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp = 0; sp < splits; ++sp) {
    const float4 v = *reinterpret_cast<const float4*>(part + (static_cast<int64_t>(sp) * rows_total + row) * N + c);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  bf16_t* op = row < max_kept ? y_perm + row * N + c : y_shared + (row - max_kept) * N + c;
  uint2 pk;
  pk.x = pack_bf16x2(s.x, s.y);
  pk.y = pack_bf16x2(s.z, s.w);
  *reinterpret_cast<uint2*>(op) = pk;
}

int max_groups(const Shape& s) {
  return static_cast<int>(std::min<int64_t>(s.E, s.T * s.k)) + s.n_shared;
}

}  // namespace

bool small_m_fits(const Shape& s) { return s.dtype == MOE_BF16 && s.T <= kSmallMMaxRows; }
bool use_small_m(const Shape& s) {
  return small_m_fits(s) && s.T * s.k < static_cast<int64_t>(kSmallMRowsPerExpert) * s.E;
}

hipError_t launch_split_reduce(const Shape& s, const float* part, int splits, const int32_t* offsets, void* y_perm,
                               void* y_shared, hipStream_t st) {
  const int64_t rows_total = s.max_kept + static_cast<int64_t>(s.n_shared) * s.T;
  const int64_t threads = rows_total * (s.d / 4);
  hipLaunchKernelGGL(small_m_reduce, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, st, part,
                     offsets, s.E, s.max_kept, s.n_shared, static_cast<int>(s.T), s.d, splits,
                     static_cast<bf16_t*>(y_perm), static_cast<bf16_t*>(y_shared));
  return hipGetLastError();
}

// K splits per launch: enough (group, chunk, split) units that the tail of the launch (the
// last, partly filled round of waves) is short, while each split keeps >= 1024 of K.
constexpr int64_t kSmallMUnitsTarget = 8192;
// wave slots of one round: 256 CUs x 2 blocks of 4 waves (two waves per SIMD)
constexpr int64_t kSmallMWaveSlots = 2048;

int small_m_splits(const Shape& s, bool gated) {
  const int fmax = s.n_shared && s.f_s > s.f ? s.f_s : s.f;
  const int64_t units = static_cast<int64_t>(max_groups(s)) * ((gated ? fmax : s.d) / 16);
  auto fits = [&](int sp) {  // every group's K splits into multiples of 64, each >= 1024
    auto ok = [&](int K) { return K % sp == 0 && (K / sp) % 64 == 0 && K / sp >= 1024; };
    if (gated) return ok(s.d);
    return ok(s.f) && (s.n_shared == 0 || ok(s.f_s));
  };
  int sp = 1;
  // a gated launch whose units all fit one round (one or two experts: a single token) runs
  // unsplit: no round tail to shorten, and no reduction launch
  if (gated && units <= kSmallMWaveSlots) return 1;
  while (units * sp < kSmallMUnitsTarget && sp < 16 && fits(2 * sp)) sp *= 2;
  return sp;
}

size_t small_m_ws_bytes(const Shape& s) {
  if (!small_m_fits(s)) return 0;  // also sized when bf16 batches take the tiled path (FP8 cannot)
  const int64_t rows_total = s.max_kept + static_cast<int64_t>(s.n_shared) * s.T;
  const int fmax = s.n_shared && s.f_s > s.f ? s.f_s : s.f;
  const int sg = small_m_splits(s, true);
  const size_t gated = sg > 1 ? static_cast<size_t>(sg) * rows_total * 2 * fmax * sizeof(float) : 0;
  const size_t down = static_cast<size_t>(small_m_splits(s, false)) * rows_total * s.d * sizeof(float);
  return align256(std::max(gated, down));
}

hipError_t launch_grouped_mlp_small(const Shape& s, const void* x, const int32_t* sorted_slot,
                                    const int32_t* offsets, const void* wg, const void* wu,
                                    const void* wd, const void* swg, const void* swu,
                                    const void* swd, void* h, void* hs, float* part,
                                    void* y_perm, void* y_shared, hipStream_t st, const Fp8Scales& fp8) {
  SmallArgs a{};
  const bool f8 = fp8.gate != nullptr;
  a.sorted_slot = sorted_slot;
  a.offsets = offsets;
  a.E = s.E;
  a.k = s.k;
  a.T = static_cast<int>(s.T);
  a.n_shared = s.n_shared;
  a.max_kept = s.max_kept;
  const int G = s.E + s.n_shared;
  // gated: h = silu(x Wg) * (x Wu)
  a.in_r = static_cast<const bf16_t*>(x);
  a.in_s = static_cast<const bf16_t*>(x);
  a.w0_r = wg;
  a.w1_r = wu;
  a.w0_s = swg;
  a.w1_s = swu;
  a.out_r = static_cast<bf16_t*>(h);
  a.out_s = static_cast<bf16_t*>(hs);
  a.N_r = s.f;
  a.K_r = s.d;
  a.N_s = s.f_s;
  a.K_s = s.d;
  const int fmax = s.n_shared && s.f_s > s.f ? s.f_s : s.f;
  a.n_chunks = fmax / 16;
  a.splits = small_m_splits(s, true);
  a.fw = fmax;
  a.part = part;
  int64_t units = static_cast<int64_t>(G) * a.n_chunks * a.splits;
  // a group holds at most T rows (an expert appears once per token; the shared expert sees T)
  const int groups16 = static_cast<int>((s.T + 15) / 16);
  const int ngw = groups16 <= 1 ? 1 : 2;
  a.halves = (groups16 + ngw - 1) / ngw;
  auto kern_g = f8 ? (ngw == 1 ? small_m_kernel<true, 1, true> : small_m_kernel<true, 2, true>)
                  : (ngw == 1 ? small_m_kernel<true, 1, false> : small_m_kernel<true, 2, false>);
  auto kern_d = f8 ? (ngw == 1 ? small_m_kernel<false, 1, true> : small_m_kernel<false, 2, true>)
                  : (ngw == 1 ? small_m_kernel<false, 1, false> : small_m_kernel<false, 2, false>);
  a.s0_r = fp8.gate;
  a.s1_r = fp8.up;
  a.s0_s = fp8.shared_gate;
  a.s1_s = fp8.shared_up;
  units *= a.halves;
  timing_begin(MOE_KERNEL_GATE_UP, st);
  hipLaunchKernelGGL(kern_g, dim3(static_cast<unsigned>((units + 3) / 4)), dim3(kThreads), 0, st, a);
  timing_end(MOE_KERNEL_GATE_UP, st);
  const int64_t rows_total = s.max_kept + static_cast<int64_t>(s.n_shared) * s.T;
  if (a.splits > 1) {
    const int64_t threads = rows_total * (fmax / 4);
    hipLaunchKernelGGL(small_m_swiglu_reduce, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, st,
                       part, offsets, s.E, s.max_kept, s.n_shared, static_cast<int>(s.T), s.f, s.f_s, fmax,
                       a.splits, static_cast<bf16_t*>(h), static_cast<bf16_t*>(hs));
  }
  // down: split-K partials, then the ordered reduction
  a.sorted_slot = nullptr;
  a.in_r = static_cast<const bf16_t*>(h);
  a.in_s = static_cast<const bf16_t*>(hs);
  a.w0_r = wd;
  a.w1_r = nullptr;
  a.s0_r = fp8.down;
  a.s1_r = nullptr;
  a.s0_s = fp8.shared_down;
  a.s1_s = nullptr;
  a.w0_s = swd;
  a.w1_s = nullptr;
  a.part = part;
  a.N_r = s.d;
  a.K_r = s.f;
  a.N_s = s.d;
  a.K_s = s.f_s;
  a.n_chunks = s.d / 16;
  a.splits = small_m_splits(s, false);
  units = static_cast<int64_t>(G) * a.n_chunks * a.splits * a.halves;
  timing_begin(MOE_KERNEL_DOWN, st);
  hipLaunchKernelGGL(kern_d, dim3(static_cast<unsigned>((units + 3) / 4)), dim3(kThreads), 0, st, a);
  timing_end(MOE_KERNEL_DOWN, st);
  if (y_perm == nullptr) return hipGetLastError();  // the caller combines from the partials
  const int64_t threads = rows_total * (s.d / 4);
  hipLaunchKernelGGL(small_m_reduce, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, st, part,
                     offsets, s.E, s.max_kept, s.n_shared, static_cast<int>(s.T), s.d, a.splits,
                     static_cast<bf16_t*>(y_perm), static_cast<bf16_t*>(y_shared));
  return hipGetLastError();
}

}  // namespace moe

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
// Work units = (token half, group slot, K split, 16-column chunk), where the group slots are
// the routed experts that hold rows (found on the device from the offsets) and then the
// shared experts, so the grid covers only what a batch of T tokens can touch (min(E, T*k)
// routed experts). K splits keep the units small, so the last, partly filled round of waves
// is short.
#include <cmath>

#include "common.h"
#include "route_block.h"

namespace moe {
namespace {

constexpr int kThreads = 256;  // at most 4 waves a block, one unit each

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
  int r_slots;                 // routed group slots: min(E, T*k), the most experts a batch can touch
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
template <bool GATED, int NG, bool FP8, int CPW = 1>
struct RingDepth {
  static constexpr int v[2] = {MOE_SM_GB1};
};
// two 16-row chunks per wave (FP8 weights, two token groups): a ring of three blocks of both
// chunks' weights and token rows fits the register file for the down launch; the gated
// launch (gate and up weights) keeps two
template <bool GATED, int NG, bool FP8>
struct RingDepth<GATED, NG, FP8, 2> {
  static constexpr int v[2] = {GATED ? 2 : 3, GATED ? 2 : 3};
};
// four chunks per wave (FP8 down launch): a ring of two blocks at two token groups (three
// spill), three at one
template <bool GATED, int NG, bool FP8>
struct RingDepth<GATED, NG, FP8, 4> {
  static constexpr int v[2] = {NG == 2 ? 2 : 3, NG == 2 ? 2 : 3};
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
// CPW: 16-row weight chunks per wave (1 or 2). With two, each token-row fragment feeds the
// multiplies of both chunks, halving the token-row reads per weight byte (which, at two token
// groups per wave, are larger than the FP8 weight reads themselves); chunk c's rows start
// c * 16 rows (cstride bytes) after chunk 0's.
// LDSP (down launch only): the fp32 partial goes to lds_part (token row tok of the unit at
// lds_part[tok * 16 * CPW + column - n0]) instead of the global partials.
template <bool GATED, int NG, bool FP8, int CPW = 1, bool LDSP = false>
__device__ __forceinline__ void small_m_unit(const SmallArgs& a, const void* w0, const void* w1,
                                             const bf16_t* const (&xp)[2], int t0, int kbeg, int kend,
                                             int quad, int l16, int M, int r0, int gi, bool shared,
                                             int N, int n0, int split, int64_t cstride = 0,
                                             float* lds_part = nullptr) {
  constexpr int NW = FP8 ? 2 : 4;  // 16-byte weight loads per lane per block and matrix
  constexpr int DW = RingDepth<GATED, NG, FP8, CPW>::v[0];
  constexpr int DX = RingDepth<GATED, NG, FP8, CPW>::v[1];
  static_assert(DX >= 1 && DW >= DX && DW % DX == 0, "the token-row ring divides the weight ring");
  struct WOps {
    u32x4 wa[CPW][NW], wb[CPW][NW];
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
  f32x4 acc0[CPW][NG], acc1[CPW][NG];
#pragma unroll
  for (int q = 0; q < CPW; ++q)
#pragma unroll
    for (int t = 0; t < NG; ++t) {
      acc0[q][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[q][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // lane covers k in [ko, ko+32) of a 128-wide block at kb: ko = kb + 32*quad, 64 contiguous
  // bytes per lane over the block's 4 loads, so every load touches both 128-byte lines of
  // each row's 256 bytes. In the 64-wide tail (`full` false) quads 2-3 read k in [kb, kb+32)
  // instead, which is in range, and the multiply zeroes what they read. Loads are issued
  // unconditionally and left untouched until their block is multiplied, so the compiler's
  // count of loads in flight stays exact and no wait drains the ring.
  auto offs = [&](int kb, bool full) { return kb + (full || quad < 2 ? quad * 32 : 0); };
  // weight bytes of chunk q's rows: k offsets in elements, chunk offsets in bytes
  auto wptr = [&](const void* base, int q, int ko, int c) -> const u32x4* {
    const char* b = static_cast<const char*>(base) + q * cstride;
    return FP8 ? reinterpret_cast<const u32x4*>(b + ko + c * 16)
               : reinterpret_cast<const u32x4*>(b + 2 * ko + c * 16);
  };
  auto load_w = [&](WOps& o, int kb, bool full) {
    const int ko = offs(kb, full);
#pragma unroll
    for (int q = 0; q < CPW; ++q)
#pragma unroll
      for (int c = 0; c < NW; ++c) {
        o.wa[q][c] = *wptr(w0, q, ko, c);
        if (GATED) o.wb[q][c] = *wptr(w1, q, ko, c);
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
      for (int q = 0; q < CPW; ++q) {
        const bf16x8 wa = wop(w.wa[q], c, m);
        bf16x8 wb{};
        if (GATED) wb = wop(w.wb[q], c, m);
#pragma unroll
        for (int t = 0; t < NG; ++t) {
          const bf16x8 x = __builtin_bit_cast(bf16x8, o.xv[t][c] & m);
          acc0[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, x, acc0[q][t], 0, 0, 0);
          if (GATED) acc1[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, x, acc1[q][t], 0, 0, 0);
        }
      }
  };
  auto mma_full = [&](const WOps& w, const XOps& o) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int q = 0; q < CPW; ++q) {
        const bf16x8 wa = wfull(w.wa[q], c);
        bf16x8 wb{};
        if (GATED) wb = wfull(w.wb[q], c);
#pragma unroll
        for (int t = 0; t < NG; ++t) {
          const bf16x8 x = __builtin_bit_cast(bf16x8, o.xv[t][c]);
          acc0[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, x, acc0[q][t], 0, 0, 0);
          if (GATED) acc1[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, x, acc1[q][t], 0, 0, 0);
        }
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
#pragma unroll
        for (int q = 0; q < CPW; ++q) {
          w.wa[q][c] = *wptr(w0, q, kw, c);
          if (GATED) w.wb[q][c] = *wptr(w1, q, kw, c);
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

  // epilogue. 16x16 C layout: lane holds weight rows n0 + 16*q + 4*quad + r (r = 0..3) of
  // chunk q for token column l16 of each group.
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    const int ncol = n0 + 16 * q + quad * 4;
    if (ncol >= N) return;
    f32x4 (&acc0q)[NG] = acc0[q];
    f32x4 (&acc1q)[NG] = acc1[q];
    if constexpr (FP8) {  // per-row scales of the FP8 weights
      const float* sc0 = shared ? a.s0_s : a.s0_r;
      const float* sc1 = shared ? a.s1_s : a.s1_r;
      const float4 s0 = *reinterpret_cast<const float4*>(sc0 + static_cast<int64_t>(gi) * N + ncol);
      const float4 s1 = GATED ? *reinterpret_cast<const float4*>(sc1 + static_cast<int64_t>(gi) * N + ncol) : s0;
  #pragma unroll
      for (int t = 0; t < NG; ++t) {
        acc0q[t] = f32x4{acc0q[t][0] * s0.x, acc0q[t][1] * s0.y, acc0q[t][2] * s0.z, acc0q[t][3] * s0.w};
        if (GATED) acc1q[t] = f32x4{acc1q[t][0] * s1.x, acc1q[t][1] * s1.y, acc1q[t][2] * s1.z, acc1q[t][3] * s1.w};
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
          *reinterpret_cast<float4*>(pp) = make_float4(acc0q[t][0], acc0q[t][1], acc0q[t][2], acc0q[t][3]);
          *reinterpret_cast<float4*>(pp + a.fw) = make_float4(acc1q[t][0], acc1q[t][1], acc1q[t][2], acc1q[t][3]);
        } else if (GATED) {
          const int64_t orow = shared ? static_cast<int64_t>(gi) * a.T + row : row;
          bf16_t* op = (shared ? a.out_s : a.out_r) + orow * N + ncol;
          uint2 pk;
          pk.x = pack_bf16x2(silu_f32(acc0q[t][0]) * acc1q[t][0], silu_f32(acc0q[t][1]) * acc1q[t][1]);
          pk.y = pack_bf16x2(silu_f32(acc0q[t][2]) * acc1q[t][2], silu_f32(acc0q[t][3]) * acc1q[t][3]);
          *reinterpret_cast<uint2*>(op) = pk;
        } else if (LDSP) {
          *reinterpret_cast<float4*>(lds_part + tok * 16 * CPW + ncol - n0) =
              make_float4(acc0q[t][0], acc0q[t][1], acc0q[t][2], acc0q[t][3]);
        } else {
          const int64_t prow = shared ? a.max_kept + static_cast<int64_t>(gi) * a.T + row : row;
          const int64_t rows_total = a.max_kept + static_cast<int64_t>(a.n_shared) * a.T;
          float* pp = a.part + (static_cast<int64_t>(split) * rows_total + prow) * N + ncol;
          *reinterpret_cast<float4*>(pp) = make_float4(acc0q[t][0], acc0q[t][1], acc0q[t][2], acc0q[t][3]);
        }
      }
    }
  }
}

// The n-th (from 0) routed group holding rows, by increasing expert index, with its first
// row and row count; g = -1 if fewer than n+1 groups hold rows. Wave-uniform: every lane
// takes part in the ballots. The offsets of up to 256 experts are loaded at once, so finding
// the group costs one memory round trip, as reading a known group's offsets does.
struct GroupRows {
  int g, r0, M;
};
__device__ __forceinline__ GroupRows nth_active_group(const int32_t* __restrict__ offsets, int E, int n, int lane) {
  int before = 0;
  for (int e0 = 0; e0 < E; e0 += 256) {
    int lo[4], hi[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // unconditional loads (clamped): no branch around them
      const int e = e0 + 64 * c + lane;
      lo[c] = offsets[min(e, E)];
      hi[c] = offsets[min(e + 1, E)];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool act = hi[c] > lo[c];
      const uint64_t m = __ballot(act);
      const int cnt = __popcll(m);
      if (n < before + cnt) {
        const int rank = __popcll(m & ((uint64_t{1} << lane) - 1));
        const uint64_t hit = __ballot(act && rank == n - before);
        const int l = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(hit)) - 1);
        const int r0 = __builtin_amdgcn_readlane(lo[c], l);
        return GroupRows{e0 + 64 * c + l, r0, __builtin_amdgcn_readlane(hi[c], l) - r0};
      }
      before += cnt;
    }
  }
  return GroupRows{-1, 0, 0};
}

// NGW: token groups of 16 per wave (1 or 2, so the 3-deep ring fits the register file). A
// group with more rows than NGW*16 is covered by `halves` passes, one per NGW token groups.
// The half is the slowest unit index: in a typical small batch every group fits one half,
// and the blocks of the other halves exit at once instead of idling inside working blocks.
// One work unit (group gr.g with rows [gr.r0, gr.r0 + gr.M) of the grouped order, K split,
// 16*CPW-column chunk nc, token half) of a wave; all indices wave-uniform. ONE_TOKEN: the
// batch is a single token, so every row gathers token 0 (no sorted_slot read).
template <bool GATED, int NGW, bool FP8, int CPW, bool LDSP = false, bool ONE_TOKEN = false>
__device__ __forceinline__ void small_m_exec(const SmallArgs& a, GroupRows gr, int nc, int split, int half,
                                             int lane, float* lds_part = nullptr) {
  const int g = gr.g;
  if (g < 0) return;  // fewer experts hold rows than there are slots
  const bool shared = g >= a.E;
  const int gi = shared ? g - a.E : g;
  const int r0 = __builtin_amdgcn_readfirstlane(gr.r0);
  const int M = __builtin_amdgcn_readfirstlane(gr.M);
  const int t0 = half * NGW;            // first token group of this wave
  const int ng = ((M + 15) >> 4) - t0;  // token groups left for it
  if (ng <= 0) return;
  const int N = shared ? a.N_s : a.N_r;
  const int K = shared ? a.K_s : a.K_r;
  const int n0 = nc * 16 * CPW;  // chunk nc: CPW 16-row chunks (N is a multiple of 64)
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
      src = GATED ? (ONE_TOKEN ? 0 : a.sorted_slot[r] / a.k) : r;
    xp[t] = in + src * K;
  }
  const int64_t cstride = int64_t{16} * K * (FP8 ? 1 : 2);  // bytes between the chunks' rows
  if (NGW == 1 || ng <= 1)
    small_m_unit<GATED, 1, FP8, CPW, LDSP>(a, w0, w1, xp, t0, kbeg, kend, quad, l16, M, r0, gi, shared, N, n0,
                                           split, cstride, lds_part);
  else
    small_m_unit<GATED, 2, FP8, CPW, LDSP>(a, w0, w1, xp, t0, kbeg, kend, quad, l16, M, r0, gi, shared, N, n0,
                                           split, cstride, lds_part);
}

// The unit of group slot gs: its group found from the offsets (slots 0 .. r_slots-1 the
// routed experts that hold rows, in increasing order; then the shared experts), then run.
template <bool GATED, int NGW, bool FP8, int CPW, bool LDSP = false>
__device__ __forceinline__ void small_m_run(const SmallArgs& a, int nc, int split, int gs, int half, int lane,
                                            float* lds_part = nullptr) {
  GroupRows gr{a.E + (gs - a.r_slots), 0, a.T};  // a shared expert: all T tokens
  if (gs < a.r_slots) {
    if (a.r_slots == a.E) {  // every expert has its slot (empty ones exit below)
      gr.g = gs;
      gr.r0 = a.offsets[gs];
      gr.M = a.offsets[gs + 1] - gr.r0;
    } else {
      gr = nth_active_group(a.offsets, a.E, gs, lane);
    }
  }
  small_m_exec<GATED, NGW, FP8, CPW, LDSP>(a, gr, nc, split, half, lane, lds_part);
}

template <bool GATED, int NGW, bool FP8, int CPW = 1>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void small_m_kernel(SmallArgs a) {
  const int lane = threadIdx.x & 63;
  // wave-uniform (readfirstlane): everything derived from the unit stays in scalar registers
  // blocks of 1 or 4 waves (blockDim.x 64 or 256)
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // unit = (half, group slot, split, chunk) with the chunk fastest: the waves of a block share
  // a group. Slots 0 .. r_slots-1 are the routed experts that hold rows, in increasing order
  // (at most min(E, T*k) of them), so no block is launched for an expert the batch does not
  // touch; the shared experts follow.
  const int GS = a.r_slots + a.n_shared;
  const int nc = static_cast<int>(unit % a.n_chunks);
  int64_t rest = unit / a.n_chunks;
  const int split = static_cast<int>(rest % a.splits);
  rest /= a.splits;
  const int gs = static_cast<int>(rest % GS);
  const int half = static_cast<int>(rest / GS);
  if (half >= a.halves) return;
  small_m_run<GATED, NGW, FP8, CPW>(a, nc, split, gs, half, lane);
}

// A single token's down launch that also combines: block nc covers the 16-column chunk nc of
// y (16 * CPW columns), one wave per (group slot, K split) unit (at most 8), bf16 or FP8
// weights. Each wave leaves its fp32 partial in LDS; then one lane per column forms y exactly
// as the ordered split reduction and the combine do
// (each kept slot's partials summed in split order and rounded to bf16, then gate-weighted
// in slot order, then the shared experts added, one rounding to bf16), so the results are
// those of the separate launches, bit for bit.
template <bool FP8, int CPW, int MAXW>
__device__ __forceinline__ void small_m_down_combine(const SmallArgs& a, const int32_t* __restrict__ pos,
                                                     const float* __restrict__ gate, bf16_t* __restrict__ y) {
  __shared__ float part[MAXW][16 * CPW];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nc = blockIdx.x;
  const int gs = w / a.splits, split = w % a.splits;
  small_m_run<false, 1, FP8, CPW, true>(a, nc, split, gs, 0, lane, part[w]);
  __syncthreads();
  if (w != 0 || lane >= 16 * CPW) return;
  auto round_bf16 = [](float v) { return __uint_as_float(pack_bf16x2(v, 0.f) << 16); };
  auto slot_sum = [&](int g) {  // the unit partials of group slot g, in split order
    float v = 0.f;
    for (int q = 0; q < a.splits; ++q) v += part[g * a.splits + q][lane];
    return round_bf16(v);
  };
  float acc = 0.f;
  for (int j = 0; j < a.k; ++j) {
    // the token's slot j: its row in the grouped order, which for a single token is the
    // group slot of its expert (every expert the token touches holds exactly that one row)
    const int p = pos[j];
    if (p < 0) continue;
    acc = fmaf(gate[j], slot_sum(p), acc);
  }
  for (int sh = 0; sh < a.n_shared; ++sh) acc += slot_sum(a.r_slots + sh);
  reinterpret_cast<uint16_t*>(y)[nc * 16 * CPW + lane] = static_cast<uint16_t>(pack_bf16x2(acc, 0.f) & 0xffffu);
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void small_m_down_combine_kernel(
    SmallArgs a, const int32_t* __restrict__ pos, const float* __restrict__ gate, bf16_t* __restrict__ y) {
  small_m_down_combine<false, 1, 8>(a, pos, gate, y);
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void small_m_down_combine_fp8_kernel(
    SmallArgs a, const int32_t* __restrict__ pos, const float* __restrict__ gate, bf16_t* __restrict__ y) {
  small_m_down_combine<true, 1, 8>(a, pos, gate, y);
}

// A single token's gated launch that routes the token itself: every block runs the block
// router on it (the first 256 threads; the same code and order as the route launch, so the
// same experts and gates), keeps its k choices in LDS, and block 0 also writes the routing
// and the permutation for the launches that follow. Then each wave runs its unit: group slot
// gs < k is the token's gs-th expert by increasing index, whose single row is row gs of the
// grouped order; the shared experts follow. Saves the route launch and its gap per step.
// Blocks of 256 to 512 threads (the block router's 256 and up to 4 more waves).
template <int EMAX, int TB, bool FP8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void small_m_routed_kernel(
    SmallArgs a, RouteArgs r) {
  __shared__ int sidx[64];
  const bool first = blockIdx.x == 0;
  router_small_e_block<bf16_t, EMAX, TB, true>(r.x, r.w_router, r.bias, r.idx, r.gate, nullptr, 1, a.K_r, a.E,
                                               a.k, r.gating, 0, sidx, first);
  __syncthreads();
  if (first && threadIdx.x < 64)
    permute_tiny_wave(sidx, a.k, a.E, r.capacity, a.max_kept, r.counts, r.offsets, r.sorted_slot, r.pos, r.drop);
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nc = unit % a.n_chunks;
  const int rest = unit / a.n_chunks;
  const int split = rest % a.splits;
  const int gs = rest / a.splits;
  if (gs >= a.r_slots + a.n_shared) return;  // past the units (the last block)
  GroupRows gr{a.E + (gs - a.r_slots), 0, 1};
  if (gs < a.r_slots) {
    // lane j < k holds choice j; its rank among the k (distinct) experts is its group slot
    const int e = lane < a.k ? sidx[lane] : 0x7fffffff;
    int rank = 0;
    for (int j = 0; j < a.k; ++j) rank += sidx[j] < e ? 1 : 0;
    const uint64_t hit = __ballot(lane < a.k && rank == gs);
    const int l = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(hit)) - 1);
    gr = GroupRows{__builtin_amdgcn_readlane(e, l), gs, 1};
  }
  small_m_exec<true, 1, FP8, 1, false, true>(a, gr, nc, split, 0, lane);
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
  float4 g, u;
  split_sum2(part + row * 2 * fw + c, rows_total * 2 * fw, fw, splits, g, u);
  bf16_t* op = routed ? h + row * f + c : hs + (row - max_kept) * f_s + c;
  uint2 pk;
  pk.x = pack_bf16x2(silu_f32(g.x) * u.x, silu_f32(g.y) * u.y);
  pk.y = pack_bf16x2(silu_f32(g.z) * u.z, silu_f32(g.w) * u.w);
  *reinterpret_cast<uint2*>(op) = pk;
}

// y = sum over splits of the partials, in split order, rounded once to bf16.
// One thread per 8 consecutive columns of one row; routed rows past N_kept are skipped.
__global__ __launch_bounds__(256) void small_m_reduce(const float* __restrict__ part,
                                                      const int32_t* __restrict__ offsets, int E,
                                                      int64_t max_kept, int n_shared, int T, int N,
                                                      int splits, bf16_t* __restrict__ y_perm,
                                                      bf16_t* __restrict__ y_shared) {
  const int64_t rows_total = max_kept + static_cast<int64_t>(n_shared) * T;
  const int co = N / 8;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows_total * co) return;
  const int64_t row = i / co;
  const int c = static_cast<int>(i % co) * 8;
  if (row < max_kept && row >= offsets[E]) return;
  float4 s0, s1;
  split_sum2(part + row * N + c, rows_total * N, 4, splits, s0, s1);
  bf16_t* op = row < max_kept ? y_perm + row * N + c : y_shared + (row - max_kept) * N + c;
  uint4 pk;
  pk.x = pack_bf16x2(s0.x, s0.y);
  pk.y = pack_bf16x2(s0.z, s0.w);
  pk.z = pack_bf16x2(s1.x, s1.y);
  pk.w = pack_bf16x2(s1.z, s1.w);
  *reinterpret_cast<uint4*>(op) = pk;
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
  const int64_t threads = rows_total * (s.d / 8);
  hipLaunchKernelGGL(small_m_reduce, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, st, part,
                     offsets, s.E, s.max_kept, s.n_shared, static_cast<int>(s.T), s.d, splits,
                     static_cast<bf16_t*>(y_perm), static_cast<bf16_t*>(y_shared));
  return hipGetLastError();
}

// K splits per launch: enough (group, chunk, split) units that the tail of the launch (the
// last, partly filled round of waves) is short, while each split keeps >= 1024 of K. A batch
// with one token group per wave that touches nearly every routed expert (so that almost no
// unit is empty) needs half as many units, and fewer splits save the reduction's partials.
// Measured A/B on the Mixtral-shaped layer (one box, interleaved), target 4096 against 8192:
// bf16 T = 16 0.514 -> 0.495 ms (gated launch unsplit), FP8 T = 16 0.297 -> 0.285 ms; but
// bf16 T = 4 (about 5.5 of the 8 experts touched) 0.325 -> 0.342 ms, and FP8 T = 64 (two token
// groups a wave) no better, so those keep 8192.
#ifndef MOE_SM_UNITS_TARGET
#define MOE_SM_UNITS_TARGET 8192
#endif
constexpr int64_t kSmallMUnitsTarget = MOE_SM_UNITS_TARGET;
constexpr int64_t kSmallMUnitsTargetFull = MOE_SM_UNITS_TARGET / 2;  // dense batches
// wave slots of one round: 256 CUs x 2 blocks of 4 waves (two waves per SIMD)
constexpr int64_t kSmallMWaveSlots = 2048;

// Waves per block of a launch of `units` work units: a launch that fits one round of wave
// slots takes blocks of one wave, so the dispatcher spreads its waves evenly over the CUs (a
// single token's gated launch: 1792 waves, 7 a CU, where blocks of four leave some CUs
// with eight and others with four; Mixtral-shaped T = 1: 85.0 -> 79.8 us); longer launches
// keep blocks of four, which dispatch faster (T = 4, 16: 1-2% slower with blocks of one).
int block_waves(int64_t units) { return units <= kSmallMWaveSlots ? 1 : 4; }

// 16-row chunks per wave of the down launch: one for bf16 weights; four for FP8 weights,
// whose token rows (bf16 h) are then read once per 64 weight rows instead of 32 (Mixtral-shaped,
// one box, A/B builds: down launch T = 64 125 -> 105 us, T = 16 87.5 -> 86.2 us, T = 4 61.3 ->
// 56.4 us), except for a single token: one chunk a wave, so that its (expert, K split) units
// of a 16-column chunk fit the one block of the down launch that also combines (two chunks
// and 8 K splits ran the separate down launch 3 us faster, but the combine launch and its gap
// cost more: FP8 T = 1 step 0.0869 -> 0.0846 ms).
int single_token_down_splits(const Shape& s, int cpw);

int small_m_down_cpw(const Shape& s, bool fp8) {
  if (!fp8) return 1;
  if (s.T > 1) return 4;
  // a single token: one chunk a wave where the down launch then combines (at most 8 units a
  // chunk), else two
  const int ts = single_token_down_splits(s, 1);
  return ts > 0 && static_cast<int64_t>(max_groups(s)) * ts <= 8 ? 1 : 2;
}

// every group's K splits into sp parts that are multiples of 64, each >= 1024
bool splits_fit(const Shape& s, bool gated, int sp) {
  auto ok = [&](int K) { return K % sp == 0 && (K / sp) % 64 == 0 && K / sp >= 1024; };
  if (gated) return ok(s.d);
  return ok(s.f) && (s.n_shared == 0 || ok(s.f_s));
}

// K splits of a single token's down launch with cpw chunks a wave, or 0 when its units do not
// fit one round of wave slots: every routed slot holds rows (the token's k experts), so the
// units are known exactly; take as many K splits as fill one round. Mixtral-shaped T = 1: 4
// splits instead of 8, down launch 47.9 -> 44.2 us.
int single_token_down_splits(const Shape& s, int cpw) {
  const int64_t real = static_cast<int64_t>(max_groups(s)) * (s.d / 16) / cpw;
  if (real > kSmallMWaveSlots) return 0;
  int sp = 1;
  while (real * 2 * sp <= kSmallMWaveSlots && sp < 16 && splits_fit(s, false, 2 * sp)) sp *= 2;
  return sp;
}

int small_m_splits(const Shape& s, bool gated, bool fp8) {
  const int fmax = s.n_shared && s.f_s > s.f ? s.f_s : s.f;
  const int64_t units = static_cast<int64_t>(max_groups(s)) * ((gated ? fmax : s.d) / 16);
  auto fits = [&](int sp) { return splits_fit(s, gated, sp); };
  int sp = 1;
  // a gated launch whose units all fit one round (one or two experts: a single token) runs
  // unsplit: no round tail to shorten, and no reduction launch
  if (gated && units <= kSmallMWaveSlots) return 1;
  if (!gated && s.T == 1) {
    const int ts = single_token_down_splits(s, small_m_down_cpw(s, fp8));
    if (ts > 0) return ts;
  }
  // expected routed experts touched by T tokens choosing k of E uniformly
  const double touched = s.E * (1.0 - std::pow(1.0 - static_cast<double>(s.k) / s.E, static_cast<double>(s.T)));
  const bool dense = s.T <= 16 && touched >= 0.95 * s.E;
  const int64_t target = dense ? kSmallMUnitsTargetFull : kSmallMUnitsTarget;
  while (units * sp < target && sp < 16 && fits(2 * sp)) sp *= 2;
  return sp;
}

// FP8 weights only: measured on the Mixtral-shaped T = 1 layer (A/B builds, interleaved, one
// box), the FP8 step went 0.0866 -> 0.0837 ms (the gated launch grows by 1 us, the route
// launch goes), while the bf16 step went 0.1340 -> 0.1350 ms (its gated launch grows by 5.5
// us: with bf16 weights the launch's blocks of seven waves stream slower than blocks of one).
bool small_m_routes(const Shape& s, bool fp8) {
  if (!fp8 || s.T != 1 || s.dtype != MOE_BF16 || s.E > 8 || s.k > s.E) return false;
  // the gated launch's units (one split: a single token's gated units fit one round)
  const int fmax = s.n_shared && s.f_s > s.f ? s.f_s : s.f;
  const int64_t units = static_cast<int64_t>(max_groups(s)) * (fmax / 16);
  return small_m_splits(s, true, true) == 1 && units <= 8LL * cu_count();
}

// The fused single-token down launch and combine: one token, at most 8 (group, K split) waves
// a 16-column chunk (small_m_down_combine_kernel, small_m_down_combine_fp8_kernel).
bool small_m_combines(const Shape& s, bool fp8) {
  if (s.T != 1 || s.dtype != MOE_BF16) return false;
  if (fp8 && small_m_down_cpw(s, true) != 1) return false;  // the fused FP8 kernel takes one chunk a wave
  return static_cast<int64_t>(max_groups(s)) * small_m_splits(s, false, fp8) <= 8;
}

size_t small_m_ws_bytes(const Shape& s) {
  if (!small_m_fits(s)) return 0;  // also sized when bf16 batches take the tiled path (FP8 cannot)
  const int64_t rows_total = s.max_kept + static_cast<int64_t>(s.n_shared) * s.T;
  const int fmax = s.n_shared && s.f_s > s.f ? s.f_s : s.f;
  const int sg = std::max(small_m_splits(s, true, false), small_m_splits(s, true, true));
  const size_t gated = sg > 1 ? static_cast<size_t>(sg) * rows_total * 2 * fmax * sizeof(float) : 0;
  const int sd = std::max(small_m_splits(s, false, false), small_m_splits(s, false, true));
  const size_t down = static_cast<size_t>(sd) * rows_total * s.d * sizeof(float);
  return align256(std::max(gated, down));
}

hipError_t launch_grouped_mlp_small(const Shape& s, const void* x, const int32_t* sorted_slot,
                                    const int32_t* offsets, const void* wg, const void* wu,
                                    const void* wd, const void* swg, const void* swu,
                                    const void* swd, void* h, void* hs, float* part,
                                    void* y_perm, void* y_shared, hipStream_t st, const Fp8Scales& fp8,
                                    const SmallCombine& comb, const RouteArgs* route) {
  SmallArgs a{};
  const bool f8 = fp8.gate != nullptr;
  a.sorted_slot = sorted_slot;
  a.offsets = offsets;
  a.E = s.E;
  a.k = s.k;
  a.T = static_cast<int>(s.T);
  a.n_shared = s.n_shared;
  a.max_kept = s.max_kept;
  a.r_slots = static_cast<int>(std::min<int64_t>(s.E, s.T * s.k));
  const int G = a.r_slots + s.n_shared;  // group slots (experts that can hold rows)
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
  // FP8 weights: two 16-row chunks per wave, so each token-row fragment feeds both and the
  // token-row reads from L2 per code byte halve. The gated launch takes them with two token
  // groups per wave (T > 16; at one group halving the units costs more than it saves), the
  // down launch always (four past a single token: small_m_down_cpw). Measured on the
  // Mixtral-shaped layer (A/B builds, one box): T = 64 gated 245 -> 203 us and down 168 ->
  // 126 us; down T = 16 104 -> 87 us; the gated launch at T <= 16 and every bf16 launch lose
  // with two chunks. The K splits are chosen on 16-column chunks either way
  // (but for a single token, see small_m_splits).
  const int groups16 = static_cast<int>((s.T + 15) / 16);
  const int cpw_g = f8 && groups16 > 1 ? 2 : 1;
  const int cpw_d = small_m_down_cpw(s, f8);
  a.n_chunks = fmax / (16 * cpw_g);
  a.splits = small_m_splits(s, true, f8);
  a.fw = fmax;
  a.part = part;
  int64_t units = static_cast<int64_t>(G) * a.n_chunks * a.splits;
  // a group holds at most T rows (an expert appears once per token; the shared expert sees T)
  const int ngw = groups16 <= 1 ? 1 : 2;
  a.halves = (groups16 + ngw - 1) / ngw;
  auto kern_g = f8 ? (ngw == 1 ? small_m_kernel<true, 1, true>
                                : (cpw_g == 2 ? small_m_kernel<true, 2, true, 2> : small_m_kernel<true, 2, true>))
                  : (ngw == 1 ? small_m_kernel<true, 1, false> : small_m_kernel<true, 2, false>);
  auto kern_d = f8 ? (ngw == 1 ? (cpw_d == 4   ? small_m_kernel<false, 1, true, 4>
                                  : cpw_d == 2 ? small_m_kernel<false, 1, true, 2>
                                               : small_m_kernel<false, 1, true, 1>)
                                : small_m_kernel<false, 2, true, 4>)  // T > 16: four chunks
                  : (ngw == 1 ? small_m_kernel<false, 1, false> : small_m_kernel<false, 2, false>);
  a.s0_r = fp8.gate;
  a.s1_r = fp8.up;
  a.s0_s = fp8.shared_gate;
  a.s1_s = fp8.shared_up;
  units *= a.halves;
  int wpb = block_waves(units);
  timing_begin(MOE_KERNEL_GATE_UP, st);
  if (route != nullptr && small_m_routes(s, f8)) {
    // a single token routed inside the launch: one block of 4 to 8 waves per CU (the block
    // router needs 256 threads), so that every block's routing is shared by its waves and
    // the waves spread evenly
    const int64_t cus = cu_count();
    const int w = std::max(4, static_cast<int>((units + cus - 1) / cus));
    auto kern = f8 ? small_m_routed_kernel<8, 4, true> : small_m_routed_kernel<8, 4, false>;  // E <= 8
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>((units + w - 1) / w)), dim3(64 * w), 0, st, a, *route);
  } else {
    hipLaunchKernelGGL(kern_g, dim3(static_cast<unsigned>((units + wpb - 1) / wpb)), dim3(64 * wpb), 0, st, a);
  }
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
  a.n_chunks = s.d / (16 * cpw_d);
  a.splits = small_m_splits(s, false, f8);
  units = static_cast<int64_t>(G) * a.n_chunks * a.splits * a.halves;
  if (comb.y != nullptr && small_m_combines(s, f8)) {
    // a single token: the down launch forms y itself, one block of G x splits waves a chunk
    timing_begin(MOE_KERNEL_DOWN, st);
    hipLaunchKernelGGL(f8 ? small_m_down_combine_fp8_kernel : small_m_down_combine_kernel,
                       dim3(static_cast<unsigned>(a.n_chunks)), dim3(static_cast<unsigned>(64 * G * a.splits)), 0, st,
                       a, comb.pos, comb.gate, static_cast<bf16_t*>(comb.y));
    timing_end(MOE_KERNEL_DOWN, st);
    return hipGetLastError();
  }
  timing_begin(MOE_KERNEL_DOWN, st);
  wpb = block_waves(units);
  hipLaunchKernelGGL(kern_d, dim3(static_cast<unsigned>((units + wpb - 1) / wpb)), dim3(64 * wpb), 0, st, a);
  timing_end(MOE_KERNEL_DOWN, st);
  if (y_perm == nullptr) return hipGetLastError();  // the caller combines from the partials
  const int64_t threads = rows_total * (s.d / 8);
  hipLaunchKernelGGL(small_m_reduce, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, st, part,
                     offsets, s.E, s.max_kept, s.n_shared, static_cast<int>(s.T), s.d, a.splits,
                     static_cast<bf16_t*>(y_perm), static_cast<bf16_t*>(y_shared));
  return hipGetLastError();
}

}  // namespace moe

// Grouped expert MLP: for every expert, its batch of gathered token rows through the
// SwiGLU block (silu(v Wg) * (v Wu)) Wd, as two grouped GEMM launches.
// Pages: klaylearn.com/glossary/mixture-of-experts, definition (one grouped GEMM over
// the batch of each expert); techbonafide.com "Mixture of Experts (MoE) Explained", section
// "Experts as Specialized Subnetworks" (an expert is a standard feed-forward block);
// shubhamtatvamasi.com/llm-inference/moe, section "The router" (a shared expert runs on every
// token, ungated).
//
// Groups: the E routed experts (rows = their slice of the grouped order, input row =
// x[sorted_slot[p] / k]) and the n_s shared experts (rows = all T tokens, identity
// gather). A device-built tile table lists (group, first row, end row) of every BM-row
// tile, so expert sizes never travel to the host and a skewed expert simply owns more
// tiles. Launch 1 (gated) computes h = silu(v Wg) * (v Wu) for a 128-column slice of f,
// with the gate and up rows of that slice side by side in LDS; launch 2 computes
// y = h Wd for a 256-column slice of d. (Batches of at most 64 tokens take the
// weight-streaming kernels of grouped_mlp_small.hip instead.)
//
// bf16 tile: 256 threads (4 waves, 2 x 2), 256 weight rows x 256 token rows, K in stages
// of 32 held in a ring of 4 LDS stages (128 KB) filled by direct-to-LDS DMA
// (global_load_lds, 16 bytes per lane) running two stages ahead of the MFMAs.
// MFMA v_mfma_f32_32x32x16_bf16 with the WEIGHT rows as operand A and the token rows as
// operand B: the accumulator then holds 4 consecutive output columns per lane, stored as
// one 8-byte write. LDS rows are 64 B; 16-byte chunk c of row r lives at chunk
// c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1), which keeps both the DMA fills and the MFMA
// operand reads (32 rows x one chunk) free of bank conflicts.
// The launch is persistent: one block per CU takes tiles from per-XCD queues.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int BW = 256;          // weight rows per tile (gated: 128 gate + 128 up)
constexpr int kTileEntries = 4;  // int32 per tile-table entry
constexpr int kQueueInts = 16;   // tile counters of the persistent launches: 8 (one per XCD) each
#ifndef MOE_GEMM_GROUP_M
#define MOE_GEMM_GROUP_M 8
#endif
constexpr int kGroupM = MOE_GEMM_GROUP_M;  // m-tiles per raster group (L2 reuse of weight tiles)
#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 32
#endif
#ifndef MOE_GEMM_NST
#define MOE_GEMM_NST (MOE_GEMM_BK == 64 ? 2 : 4)
#endif
constexpr int BK = MOE_GEMM_BK;      // K per LDS stage
constexpr int NST = MOE_GEMM_NST;    // LDS stages in the ring (stage = (256 + BT) * BK * 2 bytes)
constexpr int CH = BK / 8;               // 16-byte chunks per LDS row
constexpr int RPI = 64 / CH;             // LDS rows filled by one DMA instruction (1 KB)
constexpr int IPW = 128 / RPI;           // DMA instructions per wave per stage (128 rows)

struct GemmArgs {
  const bf16_t* in_r;          // routed input rows: x [T][K] (gather) or h [rows][K]
  const bf16_t* in_s;          // shared input rows: x [T][K] or hs [n_s*T][K]
  const int32_t* sorted_slot;  // gather for routed rows (gated launch), else nullptr
  const int32_t* tiles;        // [n][4] {group, row_begin, row_end, 0}
  const int32_t* n_tiles;      // device count of m-tiles
  const bf16_t* w0_r;          // routed weights [E][N_r][K_r] (gate, or down)
  const bf16_t* w1_r;          // routed up weights (gated)
  const bf16_t* w0_s;          // shared weights [n_s][N_s][K_s]
  const bf16_t* w1_s;
  bf16_t* out_r;               // [rows][N_r]
  bf16_t* out_s;               // [n_s*T][N_s]
  int N_r, K_r, N_s, K_s;
  int E, k, T;
  int n_tiles_n;               // n-tiles of the widest group
  int32_t* queue;              // [8] per-XCD tile counters, zeroed by build_tiles_kernel
  // weight-gradient launches (kGemmWgrad): the token operand is a transposed activation
  // [M][ld_in], the weight operand a transposed activation [N][ld_w], and a group's K range
  // is its padded segment of the columns
  const int32_t* koff;         // [E+1] first column of each routed group's segment
  int ld_in_r, ld_w_r, ld_in_s, ld_w_s;
  int64_t in_s_gstride, w_s_gstride;  // elements between consecutive shared groups
  int M_r, M_s;                // output rows of a routed / shared group
  int mt_r, mt_s, n_m;         // m-tiles of a routed / shared group, and in all
  // split-K down launch (kGemmPlainSplit): fp32 partials [splits][part_rows][N], routed rows
  // first, then shared expert s's token t at max_kept + s*T + t
  float* part;
  int splits;
  int64_t max_kept, part_rows;
  // dgrad modes: weights stored [K][N]; K rows 0..ksw-1 from w0 [E][ksw][N], the rest from
  // w1 [E][K-ksw][N]
  int ksw_r, ksw_s;
};

// Chunk swizzle of LDS row r (its 16-byte chunk c is stored at slot c ^ swz(r)). It makes
// 8 consecutive rows (32 banks) and 16 consecutive rows (64 banks) of one chunk column fall
// in distinct bank groups, for the MFMA operand reads (32 rows, one chunk) and the DMA fills
// (whole rows).
__device__ __forceinline__ int swz(int r) {
  return BK == 64 ? ((r & 7) ^ ((r >> 3) & 1)) : (((r >> 1) & 3) ^ ((r >> 3) & 1));
}

typedef __attribute__((address_space(3))) void lds_void;

// Weights stored [K][N] (the dgrad modes): a stage's weight part is BK rows of k by BW
// columns (512 B per row), 64-byte segment s of row r stored at segment s ^ tr_swz(r). A
// transposing read of a 32 x 16 operand fragment touches rows k0+{0..3} (lanes 0-31) and
// k0+{8..11} (lanes 32-63) at one segment: tr_swz sends those 8 rows to 8 distinct segments.
__device__ __forceinline__ int tr_swz(int r) { return (r & 3) | (((r >> 3) & 1) << 2); }

typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Direct-to-LDS 16-byte load (lane l's 16 bytes at g land at LDS byte address M0 + 16*l)
// issued from assembly, for the launches that read weights with ds_read_b64_tr_b16. The
// compiler's wait insertion assumes that such a read may alias any LDS DMA in flight (the
// intrinsic carries no alias information) and would drain the whole DMA ring before each
// one; hidden from it, the DMA is ordered by the K loop's own vmcnt waits and barriers,
// which are what order the plain operand reads against the DMA in every mode. The
// instruction has no register result; M0 is written here and declared clobbered, one wait
// state between the write and the load that reads it.
__device__ __forceinline__ void dma16_untracked(const char* g, const bf16_t* lds_dst) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)(lds_dst))));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(m0v) : "memory", "m0");
}

// MFMA operand fragment (column c of the fragment = lane % 32, k = 8 * (lane / 32) + 0..7)
// of a [K][N] weight stage, from p = the lane's element offset for k rows +0..3: two
// ds_read_b64_tr_b16, each of which hands lane i of a 16-lane group element i % 4 of the
// 8 bytes addressed by lane 4j + i / 4 as its element j. Lane 4j + q of a group therefore
// addresses row j, columns 4q..4q+3 of the group's 16 columns, and receives its column's
// 4 rows.
__device__ __forceinline__ bf16x8 read_tr_fragment(const bf16_t* p) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * BW));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left at their maximum (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for the K loop. __syncthreads() would also wait for every outstanding
// global access (vmcnt(0)), draining the DMA ring; here each wave has already waited for
// the stage it needs with wait_vmcnt, so only the barrier itself is issued. The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Global -> LDS fills of one stage (direct-to-LDS 16-byte loads, 1 KB per instruction).
// LDS stage layout: rows 0..BW-1 weights, BW..BW+BT-1 tokens, BK*2 bytes per row.
// Waves 0 and 1 each fill 128 weight rows, waves 2 and 3 each fill BT/2 token rows.
// Instruction i of a wave fills its rows RPI*i .. RPI*i+RPI-1: lane l stores chunk slot
// l%CH of row RPI*i + l/CH, i.e. the row's logical chunk (l%CH) ^ swz(row).
// Offsets are 32-bit byte offsets from a wave-uniform base.
// Weights stored [K][N] (TR): weight wave w fills rows w*BK/2 .. w*BK/2 + BK/2 - 1 of the
// stage, two 512-byte rows per instruction, and a stage's rows are K rows of the matrix, so
// the per-stage advance is a whole row block (step) and the dx launch switches from the gate
// to the up matrix at stage sw.
struct DmaPlan {
  const char* base;   // wave-uniform
  uint32_t off[IPW];  // byte offset of this lane's chunk for instruction i (K offset 0)
  const char* base1;  // TR: matrix read from stage sw on
  int64_t step;       // TR: bytes per stage
  int sw;             // TR: first stage read from base1

  // TR: start of stage st's rows (token waves: step = BK * 2, sw never reached)
  __device__ __forceinline__ const char* at(int st) const {
    return st < sw ? base + st * step : base1 + (st - sw) * step;
  }

  template <int BT, bool TR = false>
  __device__ __forceinline__ void issue(bf16_t* stage, int k0, int wave) const {
    static_assert(!TR || BT == 256, "TR plans fill whole stages");
    const uint32_t kb = static_cast<uint32_t>(k0) * 2u;
    if (TR) {
      const char* b = at(k0 / BK);
      bf16_t* dst = stage + wave * 128 * BK;
#pragma unroll
      for (int i = 0; i < IPW; ++i) dma16_untracked(b + off[i], dst + i * RPI * BK);
    } else if (BT == 256 || wave < 2) {
      bf16_t* dst = stage + wave * 128 * BK;
#pragma unroll
      for (int i = 0; i < IPW; ++i)
        __builtin_amdgcn_global_load_lds(base + off[i] + kb, (lds_void*)(dst + i * RPI * BK), 16, 0, 0);
    } else {
      bf16_t* dst = stage + (BW + (wave - 2) * (BT / 2)) * BK;
#pragma unroll
      for (int i = 0; i < IPW * BT / 256; ++i)
        __builtin_amdgcn_global_load_lds(base + off[i] + kb, (lds_void*)(dst + i * RPI * BK), 16, 0, 0);
    }
  }
};

// s_waitcnt lgkmcnt(0) with vmcnt and expcnt left at their maximum (gfx9 encoding).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// wait until at most `later` stages of DMA (IPW instructions each) are still in flight
__device__ __forceinline__ void wait_stages_in_flight(int later) {
  if (later >= 3) wait_vmcnt<3 * IPW>();
  else if (later == 2) wait_vmcnt<2 * IPW>();
  else if (later == 1) wait_vmcnt<IPW>();
  else wait_vmcnt<0>();
}

// Software-pipelined K loop of a 256 x 256 tile in which this wave has LIVE (0..4) token
// sub-tiles of 32 rows holding data; BK = 32, so every stage is 2 k-steps of NM = 4*LIVE
// MFMAs. Issue order per stage, pinned with scheduling barriers:
//   A: the NM MFMAs of k-step 0, interleaved with the NR = 4 + LIVE LDS reads of k-step
//      1's operands and DMA instructions kDmaC.. of stage kt+NST-1, one every 4 MFMAs;
//   B: NM/4 MFMAs of k-step 1 with the last DMA instruction;
//   -- wait for this wave's LDS reads and for stage kt+1's DMA, workgroup barrier --
//   C: the remaining MFMAs of k-step 1, interleaved with the NR reads of stage kt+1's
//      k-step 0 operands and the first kDmaC DMA instructions of stage kt+NST, whose slot
//      (that of stage kt) every wave has finished reading at the barrier.
// The 8 DMA instructions of a stage are thus spread over a whole stage's MFMAs: issued in
// a burst they fill the load queue, and an in-order wave stuck behind a full queue stops
// feeding the MFMA pipe. The barrier in the middle of the stage orders (i) every wave's
// reads of stage kt before the DMA that reuses its slot, and (ii) every wave's DMA of stage
// kt+1 before the reads of C. All waves of a block pass the same number of barriers (one
// per stage) whatever their LIVE, so waves of a ragged tile stay in step.
// TR: the weight operands come from a [K][N] stage through transposing reads (two per
// fragment, aoff = the lane's offsets of k-step 0), and the DMA addresses stage by stage.
template <int LIVE, bool TR = false>
__device__ __forceinline__ void kloop_pipelined(f32x16 (&acc)[4][LIVE > 0 ? LIVE : 1], bf16_t* lds,
                                                const DmaPlan& dp, int K, int wave,
                                                const int (&aoff)[4], const int (&boff)[LIVE > 0 ? LIVE : 1],
                                                int swz_l, int khalf) {
  constexpr int STAGE = (BW + 256) * BK;
  constexpr int NB = LIVE > 0 ? LIVE : 1;
  constexpr int NM = 4 * LIVE;            // MFMAs per k-step
  constexpr int NR = LIVE ? 4 + LIVE : 0; // LDS reads per k-step
  constexpr int MB = NM / 4;              // MFMAs of k-step 1 before the barrier
  constexpr int kDmaC = 3;                // DMA instructions of a stage issued a phase early
  const int KT = K / BK;
  bf16x8 fa0[4], fb0[NB], fa1[4], fb1[NB];
  auto rd = [&](const bf16_t* st, int kk, int idx, bf16x8 (&fa)[4], bf16x8 (&fb)[NB]) {
    const int c = ((kk * 2 + khalf) ^ swz_l) << 3;
    if (TR && idx < 4)
      fa[idx] = read_tr_fragment(st + aoff[idx] + kk * 16 * BW);
    else if (idx < 4)
      fa[idx] = *reinterpret_cast<const bf16x8*>(st + aoff[idx] + c);
    else
      fb[idx - 4] = *reinterpret_cast<const bf16x8*>(st + boff[idx - 4] + c);
  };
  auto mf = [&](int m, const bf16x8 (&fa)[4], const bf16x8 (&fb)[NB]) {
    const int i = m & 3, j = m >> 2;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  auto sb = [] { __builtin_amdgcn_sched_barrier(0); };
  // DMA instruction i of stage `st` (its slot is st % NST)
  auto dma = [&](int st, int i) {
    bf16_t* dst = lds + (st % NST) * STAGE + wave * 128 * BK;
    if constexpr (TR) {
      dma16_untracked(dp.at(st) + dp.off[i], dst + i * RPI * BK);
    } else {
      const uint32_t kb = static_cast<uint32_t>(st) * BK * 2u;
      __builtin_amdgcn_global_load_lds(dp.base + dp.off[i] + kb, (lds_void*)(dst + i * RPI * BK), 16, 0, 0);
    }
  };

  // prologue: stages 0..NST-2 in flight, wait for stage 0, fetch its k-step 0 operands,
  // then the early part of stage NST-1 (its slot has never been used)
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < KT) dp.issue<256, TR>(lds + s * STAGE, s * BK, wave);
  wait_stages_in_flight(min(NST - 2, KT - 1));
  stage_barrier();
#pragma unroll
  for (int r = 0; r < NR; ++r) rd(lds, 0, r, fa0, fb0);
  if (NST - 1 < KT) {
#pragma unroll
    for (int i = 0; i < kDmaC; ++i) dma(NST - 1, i);
  }
  sb();

  // One stage. AB: issue the rest of stage kt+NST-1 in A and B; C: the early part of stage
  // kt+NST in C; NEXT: read stage kt+1's first operands after the barrier (every stage but
  // the last). `later` = stages after kt+1 whose DMA may still be in flight at the barrier.
  auto stage_step = [&](int kt, auto ab_on, auto c_on, auto next_on, int later) {
    constexpr bool AB = decltype(ab_on)::value;
    constexpr bool DC = decltype(c_on)::value;
    constexpr bool NEXT = decltype(next_on)::value;
    const bf16_t* cur = lds + (kt % NST) * STAGE;
    // A: DMA instructions kDmaC .. kDmaC+3 after MFMAs 1, 5, 9, 13
    constexpr int NA0 = NM > NR ? NM : NR;
    constexpr int NA = NA0 > 14 ? NA0 : 14;
#pragma unroll
    for (int m = 0; m < NA; ++m) {
      if (m < NM) {
        mf(m, fa0, fb0);
        sb();
      }
      if (m < NR) {
        rd(cur, 1, m, fa1, fb1);
        sb();
      }
      if (AB && (m & 3) == 1 && (m >> 2) < 4) {
        dma(kt + NST - 1, kDmaC + (m >> 2));
        sb();
      }
    }
    // B: the last DMA instruction after the second MFMA slot
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m < MB) {
        mf(m, fa1, fb1);
        sb();
      }
      if (AB && m == 1 && kDmaC + 4 < IPW) {
        dma(kt + NST - 1, kDmaC + 4);
        sb();
      }
    }
    if (NEXT) {
      wait_lgkmcnt0();
      wait_stages_in_flight(later);
      stage_barrier();
    }
    // C: DMA instructions 0 .. kDmaC-1 of stage kt+NST after MFMAs 2, 6, 10
    const bf16_t* nxt = lds + ((kt + 1) % NST) * STAGE;
    constexpr int NC0 = NM - MB > NR ? NM - MB : NR;
    constexpr int NC = NC0 > 4 * kDmaC - 1 ? NC0 : 4 * kDmaC - 1;
#pragma unroll
    for (int m = 0; m < NC; ++m) {
      if (MB + m < NM) {
        mf(MB + m, fa1, fb1);
        sb();
      }
      if (NEXT && m < NR) {
        rd(nxt, 0, m, fa0, fb0);
        sb();
      }
      if (DC && (m & 3) == 2 && (m >> 2) < kDmaC) {
        dma(kt + NST, m >> 2);
        sb();
      }
    }
  };
  static_assert(kDmaC + 5 == IPW, "A issues 4 and B 1 of the DMA instructions after the first kDmaC");
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  int kt = 0;
  // steady state: both DMA parts every stage, NST-2 later stages in flight at each barrier
  for (; kt + NST < KT; ++kt) stage_step(kt, yes{}, yes{}, yes{}, NST - 2);
  // the stage that issues the last stage's remaining DMA
  if (kt + NST - 1 < KT) {
    stage_step(kt, yes{}, no{}, yes{}, NST - 2);
    ++kt;
  }
  // drain: no more DMA; the last stage reads nothing after it
  for (; kt + 1 < KT; ++kt) stage_step(kt, no{}, no{}, yes{}, KT - 2 - kt);
  if (kt < KT) stage_step(kt, no{}, no{}, no{}, 0);
}
static_assert(IPW == 8 || BK != 32, "the pipelined loop issues 8 DMA instructions per stage");

// Software-pipelined K loop for stages of BK = 64 (LDS rows of 128 bytes, so every DMA
// instruction fetches whole 128-byte lines, 8 rows each, and a stage takes 16 instructions a
// wave) in a ring of two stages. Per stage kt, four k-steps of NM = 4*LIVE MFMAs, operand
// fragments alternating between two register sets:
//   A: k-step 0 (set 0) | reads of k-step 1 (set 1), DMA instructions ND..15 of stage kt+1
//   B: k-step 1 (set 1) | reads of k-step 2 (set 0)
//   C: k-step 2 (set 0) | reads of k-step 3 (set 1)
//   -- wait for this wave's LDS reads and for all of stage kt+1's DMA, workgroup barrier --
//   D: k-step 3 (set 1) | reads of stage kt+1's k-step 0 (set 0), DMA instructions 0..ND-1
//      of stage kt+2 into the slot of stage kt, which every wave has finished reading
// Stage kt+2 is thus issued over D of stage kt and A of stage kt+1 and waited for at the
// barrier of stage kt+1. Both slots are filled in the prologue. Every wave passes one barrier
// per stage but the last, whatever its LIVE.
template <int LIVE>
__device__ __forceinline__ void kloop_wide(f32x16 (&acc)[4][LIVE > 0 ? LIVE : 1], bf16_t* lds,
                                           const DmaPlan& dp, int K, int wave,
                                           const int (&aoff)[4], const int (&boff)[LIVE > 0 ? LIVE : 1],
                                           int swz_l, int khalf) {
  static_assert(BK == 64 && NST == 2 && IPW == 16, "stages of 64, two of them, 16 DMA instructions a wave");
  constexpr int STAGE = (BW + 256) * BK;
  constexpr int NB = LIVE > 0 ? LIVE : 1;
  constexpr int NM = 4 * LIVE;             // MFMAs per k-step
  constexpr int NR = LIVE ? 4 + LIVE : 0;  // LDS reads per k-step
#ifndef MOE_WIDE_DMA_D
#define MOE_WIDE_DMA_D 8
#endif
  constexpr int ND = MOE_WIDE_DMA_D;       // DMA instructions of stage kt+2 issued in D
  constexpr int NA = IPW - ND;             // the rest, issued in A of the next stage
  constexpr int NMR = NM > NR ? NM : NR;
  // a phase's DMA instructions spread evenly over its MFMA slots: one every SA (SD) slots
  constexpr int SA = NA == 0 || NA >= NMR ? 1 : NMR / NA;
  constexpr int SD = ND == 0 || ND >= NMR ? 1 : NMR / ND;
  constexpr int LA = NMR > NA * SA ? NMR : NA * SA;  // slots of phase A when it issues DMA
  constexpr int LD = NMR > ND * SD ? NMR : ND * SD;
  const int KT = K / BK;
  bf16x8 fa0[4], fb0[NB], fa1[4], fb1[NB];
  auto rd = [&](const bf16_t* st, int kk, int idx, bf16x8 (&fa)[4], bf16x8 (&fb)[NB]) {
    const int c = ((kk * 2 + khalf) ^ swz_l) << 3;
    if (idx < 4)
      fa[idx] = *reinterpret_cast<const bf16x8*>(st + aoff[idx] + c);
    else
      fb[idx - 4] = *reinterpret_cast<const bf16x8*>(st + boff[idx - 4] + c);
  };
  auto mf = [&](int m, const bf16x8 (&fa)[4], const bf16x8 (&fb)[NB]) {
    const int i = m & 3, j = m >> 2;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  auto sb = [] { __builtin_amdgcn_sched_barrier(0); };
  auto dma = [&](int st, int i) {
    bf16_t* dst = lds + (st & 1) * STAGE + wave * 128 * BK;
    const uint32_t kb = static_cast<uint32_t>(st) * BK * 2u;
    __builtin_amdgcn_global_load_lds(dp.base + dp.off[i] + kb, (lds_void*)(dst + i * RPI * BK), 16, 0, 0);
  };

  // prologue: both slots filled, wait for stage 0, read its k-step 0 operands
#pragma unroll
  for (int i = 0; i < IPW; ++i) dma(0, i);
  if (KT > 1) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) dma(1, i);
    wait_vmcnt<IPW>();
  } else {
    wait_vmcnt<0>();
  }
  stage_barrier();
#pragma unroll
  for (int r = 0; r < NR; ++r) rd(lds, 0, r, fa0, fb0);
  sb();

  // A_ON: A issues the second half of stage kt+1; D_ON: D issues the first half of stage kt+2;
  // NEXT: the barrier and the reads of stage kt+1 (every stage but the last)
  auto stage_step = [&](int kt, auto a_on, auto d_on, auto next_on) {
    constexpr bool A_ON = decltype(a_on)::value;
    constexpr bool D_ON = decltype(d_on)::value;
    constexpr bool NEXT = decltype(next_on)::value;
    const bf16_t* cur = lds + (kt & 1) * STAGE;
    // A: a DMA instruction after every second MFMA slot
#pragma unroll
    for (int m = 0; m < (A_ON ? LA : NMR); ++m) {
      if (m < NM) {
        mf(m, fa0, fb0);
        sb();
      }
      if (m < NR) {
        rd(cur, 1, m, fa1, fb1);
        sb();
      }
      if (A_ON && m % SA == SA - 1 && m / SA < NA) {
        dma(kt + 1, ND + m / SA);
        sb();
      }
    }
    // B
#pragma unroll
    for (int m = 0; m < NMR; ++m) {
      if (m < NM) {
        mf(m, fa1, fb1);
        sb();
      }
      if (m < NR) {
        rd(cur, 2, m, fa0, fb0);
        sb();
      }
    }
    // C
#pragma unroll
    for (int m = 0; m < NMR; ++m) {
      if (m < NM) {
        mf(m, fa0, fb0);
        sb();
      }
      if (m < NR) {
        rd(cur, 3, m, fa1, fb1);
        sb();
      }
    }
    if (NEXT) {
      wait_lgkmcnt0();
      wait_vmcnt<0>();
      stage_barrier();
    }
    // D: a DMA instruction before every second MFMA slot
    const bf16_t* nxt = lds + ((kt + 1) & 1) * STAGE;
#pragma unroll
    for (int m = 0; m < (D_ON ? LD : NMR); ++m) {
      if (D_ON && m % SD == 0 && m / SD < ND) {
        dma(kt + 2, m / SD);
        sb();
      }
      if (m < NM) {
        mf(m, fa1, fb1);
        sb();
      }
      if (NEXT && m < NR) {
        rd(nxt, 0, m, fa0, fb0);
        sb();
      }
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  if (KT >= 3)
    stage_step(0, no{}, yes{}, yes{});
  else if (KT == 2)
    stage_step(0, no{}, no{}, yes{});
  else
    stage_step(0, no{}, no{}, no{});
  int kt = 1;
  for (; kt + 2 < KT; ++kt) stage_step(kt, yes{}, yes{}, yes{});
  if (kt == KT - 2) {
    stage_step(kt, yes{}, no{}, yes{});
    ++kt;
  }
  if (kt == KT - 1) stage_step(kt, no{}, no{}, no{});
}

// K loop and epilogue of one wave, for LIVE (compile-time) token sub-tiles of 32 rows that
// hold data. Every wave of a block runs the same number of K steps and barriers; waves
// with fewer live sub-tiles skip MFMAs, not loads.
template <bool GATED, int BT, int LIVE, bool SAVE = false, bool F32 = false, bool TR = false>
__device__ __forceinline__ void tile_loop(bf16_t* lds, const DmaPlan& dp, int K, int wave,
                                          int lane, int row0, int row1, int n0, int N,
                                          void* out_v, int64_t out_row_base) {
  constexpr int STAGE = (BW + BT) * BK;  // bf16 elements per stage
  const int wn = wave & 1, wm = wave >> 1;
  const int l32 = lane & 31, khalf = lane >> 5;
  // token sub-tile j of this wave = 32-row sub-tile 2j + wm of the tile: the two wave pairs
  // alternate, so a partly filled tile splits its live rows between them
  const int swz_l = swz(l32);  // every row a lane reads is l32 + a multiple of 32
  // LDS element offsets of this lane's operand rows
  int aoff[4], boff[LIVE > 0 ? LIVE : 1];
  static_assert(!(TR && GATED), "the [K][N] weight layout is read by the plain modes only");
  if constexpr (TR) {
    // transposing reads of the [K][N] stage: lane 4j + q of 16-lane group g addresses row
    // 8*khalf + j (+4 for the second read), columns 16*(g & 1) + 4q.. of the fragment
    const int j = (lane & 15) >> 2, q = lane & 3, hh = (lane >> 4) & 1;
    const int fl = tr_swz(8 * khalf + j);  // the same for every row this lane reads
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = (8 * khalf + j) * BW + (((wn * 4 + i) ^ fl) << 5) + 16 * hh + 4 * q;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      aoff[i] = ((GATED ? (i < 2 ? 0 : BW / 2) + wn * 64 + (i & 1) * 32 : wn * 128 + i * 32) + l32) * BK;
  }
#pragma unroll
  for (int j = 0; j < LIVE; ++j) boff[j] = (BW + (2 * j + wm) * 32 + l32) * BK;

  f32x16 acc[4][LIVE > 0 ? LIVE : 1];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < LIVE; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  constexpr int NB = LIVE > 0 ? LIVE : 1;
  auto fetch = [&](const bf16_t* stage, int kk, bf16x8 (&af)[4], bf16x8 (&bf)[NB]) {
    const int c = ((kk * 2 + khalf) ^ swz_l) << 3;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = TR ? read_tr_fragment(stage + aoff[i] + kk * 16 * BW) : *reinterpret_cast<const bf16x8*>(stage + aoff[i] + c);
#pragma unroll
    for (int j = 0; j < LIVE; ++j) bf[j] = *reinterpret_cast<const bf16x8*>(stage + boff[j] + c);
  };
  auto mma = [&](const bf16x8 (&af)[4], const bf16x8 (&bf)[NB]) {
#pragma unroll
    for (int j = 0; j < LIVE; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
  };
  // BK/16 k-steps of 16 per stage; operand fragments alternate between two register sets
  // so the LDS reads of step kk+1 can be in flight while the MFMAs of step kk run
  auto compute = [&](const bf16_t* stage) {
    if (LIVE == 0) return;
    bf16x8 a0[4], b0[NB], a1[4], b1[NB];
    fetch(stage, 0, a0, b0);
    fetch(stage, 1, a1, b1);
    mma(a0, b0);
    if (BK == 64) fetch(stage, 2, a0, b0);
    mma(a1, b1);
    if (BK == 64) {
      fetch(stage, 3, a1, b1);
      mma(a0, b0);
      mma(a1, b1);
    }
  };
  static_assert(BK == 64 || BK == 32, "compute() walks 2 or 4 k-steps of 16");

  if constexpr (BT == 256 && BK == 32 && NST >= 3) {
    kloop_pipelined<LIVE, TR>(acc, lds, dp, K, wave, aoff, boff, swz_l, khalf);
  } else if constexpr (BT == 256 && BK == 64 && NST == 2 && !TR) {
    kloop_wide<LIVE>(acc, lds, dp, K, wave, aoff, boff, swz_l, khalf);
  } else {
    // Ring of NST LDS stages, DMA running NST-1 stages ahead of the MFMAs. At step kt the
    // stage kt is complete once at most (NST-2) later stages of DMA are still in flight.
    // (one back-edge and no early exit keeps the accumulators in place across iterations)
    const int KT = K / BK;
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
      if (s < KT) dp.issue<BT, TR>(lds + s * STAGE, s * BK, wave);
    for (int kt = 0; kt < KT; ++kt) {
      // DMA instructions per stage: IPW, or IPW*BT/256 for token waves of a BT < 256 tile
      if (kt + NST - 2 >= KT)
        wait_vmcnt<0>();
      else if (BT == 256 || wave < 2)
        wait_vmcnt<(NST - 2) * IPW>();
      else
        wait_vmcnt<(NST - 2) * IPW * BT / 256>();
      stage_barrier();
      const int nxt = kt + NST - 1;
      if (nxt < KT) dp.issue<BT, TR>(lds + (nxt % NST) * STAGE, nxt * BK, wave);
      compute(lds + (kt % NST) * STAGE);
    }
  }

  // epilogue. fp32 split partials are stored straight from the accumulators; bf16 products go
  // out through LDS (measured per tile: staging takes the plain epilogue from 15 k to 10 k
  // cycles and the weight-gradient one from 21 k to 12 k, but costs the fp32 one 10% more;
  // for the gated launch's h it measured 8% slower while the read-back alternated LDS reads
  // and stores, and 0.5-1% faster with the batched read-back and non-temporal stores:
  // DeepSeek-shaped gated launch 8.44 -> 8.39 ms, Mixtral 1.703 -> 1.685 ms).
  constexpr bool STAGED = !F32;
  if constexpr (!STAGED) {
    // epilogue. acc[i][j] register r of lane l: weight row (operand A) 8*(r/4) + 4*(l/32) + r%4
    // of sub-tile i, token row 32*(2j + wm) + l%32.
  #pragma unroll
    for (int j = 0; j < LIVE; ++j) {
      const int row = row0 + (2 * j + wm) * 32 + l32;
      if (row >= row1) continue;
      // SAVE: the gate and up products themselves, side by side in a row of 2N; F32: fp32 sums
      bf16_t* op = static_cast<bf16_t*>(out_v) + (out_row_base + row) * (SAVE ? 2 * N : N);
      if (!GATED && F32) {
        float* opf = static_cast<float*>(out_v) + (out_row_base + row) * N;
  #pragma unroll
        for (int i = 0; i < 4; ++i)
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn * 128 + i * 32 + q * 8 + khalf * 4;
            if (n < N)
              *reinterpret_cast<float4*>(opf + n) =
                  make_float4(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1], acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
          }
      } else if (GATED && SAVE) {
  #pragma unroll
        for (int i = 0; i < 2; ++i)
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn * 64 + i * 32 + q * 8 + khalf * 4;
            if (n < N) {
              uint2 pa, pb;
              pa.x = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
              pa.y = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
              pb.x = pack_bf16x2(acc[i + 2][j][q * 4 + 0], acc[i + 2][j][q * 4 + 1]);
              pb.y = pack_bf16x2(acc[i + 2][j][q * 4 + 2], acc[i + 2][j][q * 4 + 3]);
              *reinterpret_cast<uint2*>(op + n) = pa;
              *reinterpret_cast<uint2*>(op + N + n) = pb;
            }
          }
      } else if (GATED) {
  #pragma unroll
        for (int i = 0; i < 2; ++i)
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn * 64 + i * 32 + q * 8 + khalf * 4;
            if (n < N) {
              float h[4];
  #pragma unroll
              for (int u = 0; u < 4; ++u) {
                const float gv = acc[i][j][q * 4 + u];
                const float uv = acc[i + 2][j][q * 4 + u];
                h[u] = silu_f32(gv) * uv;
              }
              uint2 pk;
              pk.x = pack_bf16x2(h[0], h[1]);
              pk.y = pack_bf16x2(h[2], h[3]);
              *reinterpret_cast<uint2*>(op + n) = pk;
            }
          }
      } else {
  #pragma unroll
        for (int i = 0; i < 4; ++i)
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn * 128 + i * 32 + q * 8 + khalf * 4;
            if (n < N) {
              uint2 pk;
              pk.x = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
              pk.y = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
              *reinterpret_cast<uint2*>(op + n) = pk;
            }
          }
      }
    }
  } else {
    // epilogue. acc[i][j] register r of lane l holds weight row (operand A) 8*(r/4) + 4*(l/32)
    // + r%4 of sub-tile i and token row 32*(2j + wm) + l%32: a lane has 4 consecutive output
    // columns of one token row, so a store straight from the registers touches 32 rows (32
    // cache lines, 8 or 16 bytes each). Instead each wave stages its outputs in its own quarter
    // of the stage ring, idle now, as token rows of its output columns (16-byte chunks
    // XOR-swizzled by row), and reads back whole 16-byte chunks of a row per lane: a store
    // instruction then writes 64 / CHR rows, each a contiguous CHR*16-byte segment.
    // F32 (split partials, 512-byte rows) goes through in passes of SPP sub-tiles.
    constexpr int CW = GATED && !SAVE ? 64 : 128;       // output columns of this wave
    constexpr int ES = F32 ? 4 : 2;                     // bytes per output element
    constexpr int CHR = CW * ES / 16;                   // 16-byte chunks per staged row: 8, 16, 32
    constexpr int TJL = BT / 64;                        // token sub-tiles per wave
    constexpr int SPP = F32 ? (BT == 256 ? 2 : 1) : TJL;  // token sub-tiles per pass
    constexpr int QUARTER = BT == 256 ? 32768 : BT == 128 ? 16384 : 8192;  // bytes of the ring per wave
    static_assert(SPP * 32 * CHR * 16 <= QUARTER, "a pass fits the wave's quarter of the ring");
    static_assert(4 * QUARTER <= NST * (BW + BT) * BK * 2, "the quarters fit the ring");
    stage_barrier();  // every wave is done reading the last stage
    char* stg = reinterpret_cast<char*>(lds) + wave * QUARTER;
    // an opaque copy of the lane index: the staging addresses depend on the lane only, and
    // the compiler would otherwise hoist all of them out of the persistent tile loop, keeping
    // ~70 registers live through every K loop (and spilling)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int el32 = ln & 31, ekh = ln >> 5;
    const int ld_out = SAVE ? 2 * N : N;
  #pragma unroll
    for (int p0 = 0; p0 < LIVE; p0 += SPP) {
      // stage sub-tiles p0 .. p0+SPP-1 (those < LIVE): row lr = 32*(j - p0) + l%32
  #pragma unroll
      for (int j = p0; j < p0 + SPP && j < LIVE; ++j) {
        const int lr = (j - p0) * 32 + el32;
        char* srow = stg + lr * (CHR * 16);
        auto put8 = [&](int chunk, uint2 v) {  // 8 bytes at half khalf of a 16-byte chunk
          *reinterpret_cast<uint2*>(srow + ((chunk ^ (lr & (CHR - 1))) << 4) + ekh * 8) = v;
        };
        if constexpr (F32) {
  #pragma unroll
          for (int i = 0; i < 4; ++i)
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int chunk = i * 8 + q * 2 + ekh;  // columns i*32 + q*8 + khalf*4 .. +3
              *reinterpret_cast<float4*>(srow + ((chunk ^ (lr & (CHR - 1))) << 4)) =
                  make_float4(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1], acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
            }
        } else if constexpr (GATED && SAVE) {
  #pragma unroll
          for (int i = 0; i < 2; ++i)
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint2 pa, pb;
              pa.x = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
              pa.y = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
              pb.x = pack_bf16x2(acc[i + 2][j][q * 4 + 0], acc[i + 2][j][q * 4 + 1]);
              pb.y = pack_bf16x2(acc[i + 2][j][q * 4 + 2], acc[i + 2][j][q * 4 + 3]);
              put8(i * 4 + q, pa);      // gate products: chunks 0..7
              put8(8 + i * 4 + q, pb);  // up products: chunks 8..15
            }
        } else if constexpr (GATED) {
  #pragma unroll
          for (int i = 0; i < 2; ++i)
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              float h[4];
  #pragma unroll
              for (int u = 0; u < 4; ++u) h[u] = silu_f32(acc[i][j][q * 4 + u]) * acc[i + 2][j][q * 4 + u];
              uint2 pk;
              pk.x = pack_bf16x2(h[0], h[1]);
              pk.y = pack_bf16x2(h[2], h[3]);
              put8(i * 4 + q, pk);
            }
        } else {
  #pragma unroll
          for (int i = 0; i < 4; ++i)
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint2 pk;
              pk.x = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
              pk.y = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
              put8(i * 4 + q, pk);
            }
        }
      }
      // read back: lane l takes chunk l % CHR of staged row it*(64/CHR) + l/CHR, eight rows
      // of instructions at a time (reads, then stores: one LDS latency per eight stores)
      constexpr int RPIT = 64 / CHR;  // staged rows per instruction
      constexpr int NIT = SPP * 32 / RPIT;
      constexpr int RB = NIT < 8 ? NIT : 8;
      const int rows = (min(LIVE, p0 + SPP) - p0) * 32;
  #pragma unroll
      for (int it0 = 0; it0 < NIT; it0 += RB) {
        if (it0 * RPIT >= rows) break;
        uint4 vb[RB];
  #pragma unroll
        for (int u = 0; u < RB; ++u) {
          const int lr = (it0 + u) * RPIT + ln / CHR;
          const int c = ln % CHR;
          if ((it0 + u) * RPIT < rows)
            vb[u] = *reinterpret_cast<const uint4*>(stg + lr * (CHR * 16) + ((c ^ (lr & (CHR - 1))) << 4));
        }
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int it = it0 + u;
        const int lr = it * RPIT + ln / CHR;
        if (it * RPIT >= rows) break;
        const int c = ln % CHR;
        const uint4 v = vb[u];
        const int jt = p0 + lr / 32;  // this wave's sub-tile
        const int row = row0 + (2 * jt + wm) * 32 + (lr & 31);
        if (row >= row1) continue;
        if constexpr (F32) {
          const int n = n0 + wn * 128 + c * 4;
          if (n < N)
            *reinterpret_cast<uint4*>(static_cast<float*>(out_v) + (out_row_base + row) * N + n) = v;
        } else {
          bf16_t* op = static_cast<bf16_t*>(out_v) + (out_row_base + row) * ld_out;
          int n, col;
          if constexpr (GATED && SAVE) {
            n = n0 + wn * 64 + (c & 7) * 8;
            col = c < 8 ? n : N + n;
          } else if constexpr (GATED) {
            n = n0 + wn * 64 + c * 8;
            col = n;
          } else {
            n = n0 + wn * 128 + c * 8;
            col = n;
          }
          // non-temporal: each store writes whole 256-byte row segments that no later part of
          // the launch reads (down launch 0.6-2% faster; the gated launch's 16-byte pieces of h
          // were 6-14% slower with it, so they keep ordinary stores)
          if (n < N) __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4v*>(op + col));
        }
      }
      }
    }
  }
}

// Raster run of m-tile i of a group whose n m-tiles start at m-tile `first`: the group's
// m-tiles in ceil(n / kGroupM) runs of near-equal size (9 -> 5 + 4), so that the tiles an XCD
// runs at once share one group's weight tiles. Encoded as run start | run size << 24.
__device__ __forceinline__ int32_t raster_run(int first, int n, int i) {
  const int nc = (n + kGroupM - 1) / kGroupM;
  const int base = n / nc, rem = n % nc;  // rem runs of base + 1, then runs of base
  int start, size;
  if (i < rem * (base + 1)) {
    start = (i / (base + 1)) * (base + 1);
    size = base + 1;
  } else {
    start = rem * (base + 1) + ((i - rem * (base + 1)) / base) * base;
    size = base;
  }
  return (first + start) | (size << 24);
}

// One tile: BW weight rows x BT token rows, 4 waves as 2 (weights) x 2 (tokens), each
// wave 128 weight rows x BT/2 tokens (alternate 32-row sub-tiles) of
// v_mfma_f32_32x32x16_bf16 accumulators. L is the
// tile's index in raster order: groups of kGroupM m-tiles sweep every n-tile, so a weight
// tile is read by kGroupM m-tiles close together in time.
// MODE (GemmMode): the forward launches (gated with the SiLU*mul epilogue; plain), the
// gated launch storing both products (kGemmGatedSave), the weight-gradient launch
// (kGemmWgrad, fixed M rows per group, K = the group's segment), and the dgrad launches,
// whose weights are stored [K][N] (the forward's matrices read along their output index,
// no transposed copy): kGemmDgradGather gathers its routed rows by sorted_slot as the gated
// launch does, kGemmDgrad / kGemmDgradSplit read rows as kGemmPlain does.
template <int MODE, int BT>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, bf16_t* lds, int L, int n_m, int n_n) {
  constexpr bool GATED = MODE == kGemmGated || MODE == kGemmGatedSave;
  constexpr bool SAVE = MODE == kGemmGatedSave;
  constexpr bool GATHER = GATED || MODE == kGemmDgradGather;
  constexpr bool WGRAD = MODE == kGemmWgrad;
  constexpr bool SPLIT = MODE == kGemmPlainSplit || MODE == kGemmDgradSplit;
  constexpr bool TR = MODE == kGemmDgradGather || MODE == kGemmDgrad || MODE == kGemmDgradSplit;
  constexpr int WT = BT / 2;  // token rows per wave
  constexpr int TJ = WT / 32; // token sub-tiles per wave
  int split = 0;
  if constexpr (SPLIT) {  // the split is the slowest index: each split sweeps the tiles in raster order
    const int per = n_m * n_n;
    split = L / per;
    L -= split * per;
  }
  // raster groups: runs of m-tiles that sweep every n-tile together. A run of s m-tiles
  // starting at m-tile f owns the tiles L in [f*n_n, (f+s)*n_n), so L / n_n is one of its
  // m-tiles, which names the run: entry 3 of its tile-table entry (f | s << 24), or, for the
  // weight-gradient launches (a fixed mt_r / mt_s m-tiles per group), the same chunking
  // computed in place
  int run;
  const int q = L / n_n;
  if constexpr (WGRAD) {
    const int routed_m = a.E * a.mt_r;
    if (q < routed_m) {
      const int i = q % a.mt_r;
      run = raster_run(q - i, a.mt_r, i);
    } else {
      const int i = (q - routed_m) % a.mt_s;
      run = raster_run(q - i, a.mt_s, i);
    }
  } else {
    run = a.tiles[q * kTileEntries + 3];
  }
  run = __builtin_amdgcn_readfirstlane(run);
  const int first_m = run & 0xFFFFFF;
  const int gsz = run >> 24;
  const int local = L - first_m * n_n;
  const int m_idx = first_m + local % gsz;
  const int n_tile = local / gsz;

  // tile bookkeeping is wave-uniform: keep it in scalar registers
  int g, row0, row1;
  if constexpr (WGRAD) {
    const int routed_m = a.E * a.mt_r;
    if (m_idx < routed_m) {
      g = m_idx / a.mt_r;
      row0 = (m_idx % a.mt_r) * BT;
      row1 = min(row0 + BT, a.M_r);
    } else {
      g = a.E + (m_idx - routed_m) / a.mt_s;
      row0 = ((m_idx - routed_m) % a.mt_s) * BT;
      row1 = min(row0 + BT, a.M_s);
    }
    g = __builtin_amdgcn_readfirstlane(g);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    row1 = __builtin_amdgcn_readfirstlane(row1);
  } else {
    g = __builtin_amdgcn_readfirstlane(a.tiles[m_idx * kTileEntries + 0]);
    row0 = __builtin_amdgcn_readfirstlane(a.tiles[m_idx * kTileEntries + 1]);
    row1 = __builtin_amdgcn_readfirstlane(a.tiles[m_idx * kTileEntries + 2]);
  }
  const bool shared = g >= a.E;
  const int N = shared ? a.N_s : a.N_r;
  constexpr int BNO = GATED ? BW / 2 : BW;  // output columns per tile
  const int n0 = n_tile * BNO;
  if (n0 >= N) return;
  const int gi = shared ? g - a.E : g;
  int K, ldw, ldin;
  int kstart = 0, ksw = 0;  // TR: first K row of this launch's range, first row of w1
  const bf16_t* w0;
  const bf16_t* w1 = nullptr;
  const bf16_t* in;
  if constexpr (WGRAD) {
    // opaque copies: a select between two of these kernel-argument fields is otherwise
    // folded into an indexed access of a scratch copy of the arguments
    int lw_r = a.ld_w_r, lw_s = a.ld_w_s, li_r = a.ld_in_r, li_s = a.ld_in_s;
    asm volatile("" : "+s"(lw_r), "+s"(lw_s), "+s"(li_r), "+s"(li_s));
    if (shared) {
      K = a.K_s;
      w0 = a.w0_s + gi * a.w_s_gstride;
      in = a.in_s + gi * a.in_s_gstride;
      ldw = lw_s;
      ldin = li_s;
    } else {
      const int k0 = __builtin_amdgcn_readfirstlane(a.koff[g]);
      K = __builtin_amdgcn_readfirstlane(a.koff[g + 1]) - k0;
      w0 = a.w0_r + k0;
      in = a.in_r + k0;
      ldw = lw_r;
      ldin = li_r;
    }
  } else if constexpr (TR) {
    // this group's matrices: w0 [ksw][N], w1 [K-ksw][N]; rows of K are rows of memory
    int ksw_r = a.ksw_r, ksw_s = a.ksw_s;
    asm volatile("" : "+s"(ksw_r), "+s"(ksw_s));
    K = shared ? a.K_s : a.K_r;
    ksw = shared ? ksw_s : ksw_r;
    w0 = (shared ? a.w0_s : a.w0_r) + static_cast<int64_t>(gi) * ksw * N;
    w1 = (shared ? a.w1_s : a.w1_r) + static_cast<int64_t>(gi) * (K - ksw) * N;
    in = shared ? a.in_s : a.in_r;
    ldw = N;
    ldin = K;
    if constexpr (SPLIT) {
      const int ks = K / a.splits;
      kstart = split * ks;
      in += kstart;
      K = ks;
    }
  } else {
    K = shared ? a.K_s : a.K_r;
    w0 = (shared ? a.w0_s : a.w0_r) + static_cast<int64_t>(gi) * N * K;
    if (GATED) w1 = (shared ? a.w1_s : a.w1_r) + static_cast<int64_t>(gi) * N * K;
    in = shared ? a.in_s : a.in_r;
    ldw = K;
    ldin = K;
    if constexpr (SPLIT) {  // this split's K range; rows keep their full stride
      const int ks = K / a.splits;
      w0 += split * ks;
      in += split * ks;
      K = ks;
    }
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- DMA plan: waves 0-1 fill the weight rows, waves 2-3 the token rows. Rows past the
  // end (weights past N, tokens past row1) re-read a valid row; their results are dropped.
  DmaPlan dp;
  const int lrow = lane / CH;  // row within an instruction's RPI rows
  if (TR) {  // token waves advance BK columns a stage and never switch matrices
    dp.step = BK * 2;
    dp.sw = 0x7fffffff;
    dp.base1 = nullptr;
  }
  if (TR && wave < 2) {
    // [K][N] weights: instruction i of weight wave w fills stage rows R = w*BK/2 + 2i + lane/32
    // (K rows kstart + st*BK + R), 16-byte slot lane%32 of the row, i.e. columns
    // n0 + 32*((slot/4) ^ tr_swz(R)) + 8*(slot%4). Columns past N re-read column N-8.
    const int sl = lane & 31;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r = wave * (BK / 2) + 2 * i + (lane >> 5);
      const int col = min(n0 + (((sl >> 2) ^ tr_swz(r)) << 5) + ((sl & 3) << 3), N - 8);
      dp.off[i] = static_cast<uint32_t>(r) * static_cast<uint32_t>(ldw) * 2u + static_cast<uint32_t>(col) * 2u;
    }
    dp.step = static_cast<int64_t>(BK) * ldw * 2;
    if (kstart >= ksw) {  // the whole range lies in w1
      dp.base = reinterpret_cast<const char*>(w1 + static_cast<int64_t>(kstart - ksw) * ldw);
      dp.sw = 0x7fffffff;
    } else {
      dp.base = reinterpret_cast<const char*>(w0 + static_cast<int64_t>(kstart) * ldw);
      dp.base1 = reinterpret_cast<const char*>(w1);
      dp.sw = (ksw - kstart) / BK;
    }
  } else if (wave < 2) {
    // gated: wave 0 the 128 gate rows, wave 1 the 128 up rows; else 128 rows each
    const bf16_t* wb = GATED ? (wave == 0 ? w0 : w1) : w0;
    const int nbase = GATED ? n0 : n0 + wave * 128;
    dp.base = reinterpret_cast<const char*>(wb);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r = i * RPI + lrow;  // row within the wave's 128 (row mod 128 fixes the swizzle)
      const int n = min(nbase + r, N - 1);
      const int c = (lane % CH) ^ swz(r);
      dp.off[i] = static_cast<uint32_t>(n) * static_cast<uint32_t>(ldw) * 2u + (c << 4);
    }
  } else {
    dp.base = reinterpret_cast<const char*>(in);
    int rr[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r = row0 + (wave - 2) * WT + i * RPI + lrow;  // row0 + token row within the tile
      rr[i] = r < row1 ? r : row0;
    }
    if (GATHER && !WGRAD && !shared) {
      // gathered rows: all the slot loads first, so their latencies overlap (in source
      // order the compiler waits for each before issuing the next)
      uint32_t sl[IPW];
#pragma unroll
      for (int i = 0; i < IPW; ++i) sl[i] = static_cast<uint32_t>(a.sorted_slot[rr[i]]);
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t kk = static_cast<uint32_t>(a.k);
#pragma unroll
      for (int i = 0; i < IPW; ++i) rr[i] = static_cast<int>(sl[i] / kk);
    }
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int tr = (wave - 2) * WT + i * RPI + lrow;  // token row within the tile
      int64_t src = rr[i];
      if (!WGRAD && shared && !GATHER) src += static_cast<int64_t>(gi) * a.T;
      const int c = (lane % CH) ^ swz(BW + tr);
      dp.off[i] = static_cast<uint32_t>(src * ldin * 2 + (c << 4));
    }
  }

  void* out = SPLIT ? static_cast<void*>(a.part) : static_cast<void*>(shared ? a.out_s : a.out_r);
  int64_t out_row_base;
  if constexpr (WGRAD)
    out_row_base = static_cast<int64_t>(gi) * (shared ? a.M_s : a.M_r);
  else if constexpr (SPLIT)
    out_row_base = split * a.part_rows + (shared ? a.max_kept + static_cast<int64_t>(gi) * a.T : 0);
  else
    out_row_base = shared ? static_cast<int64_t>(gi) * a.T : 0;
  // live token sub-tiles of this wave: those of the tile's ceil(rows/32) that are 2j + wm
  const int sub = (row1 - row0 + 31) / 32;
  const int live = __builtin_amdgcn_readfirstlane(max(0, min(TJ, (sub - (wave >> 1) + 1) / 2)));
  static_assert(TJ == 4 || TJ == 2 || TJ == 1, "token sub-tiles per wave");
  if (live >= TJ)
    tile_loop<GATED, BT, TJ, SAVE, SPLIT, TR>(lds, dp, K, wave, lane, row0, row1, n0, N, out, out_row_base);
  else if (live == 0)
    tile_loop<GATED, BT, 0, SAVE, SPLIT, TR>(lds, dp, K, wave, lane, row0, row1, n0, N, out, out_row_base);
  else if (live == 1)
    tile_loop<GATED, BT, 1, SAVE, SPLIT, TR>(lds, dp, K, wave, lane, row0, row1, n0, N, out, out_row_base);
  else if (TJ == 4 && live == 2)
    tile_loop<GATED, BT, (TJ == 4 ? 2 : 1), SAVE, SPLIT, TR>(lds, dp, K, wave, lane, row0, row1, n0, N, out, out_row_base);
  else
    tile_loop<GATED, BT, (TJ == 4 ? 3 : 1), SAVE, SPLIT, TR>(lds, dp, K, wave, lane, row0, row1, n0, N, out, out_row_base);
}

// Persistent launch: one block per CU takes tiles from queues until all are done. The
// tiles in raster order are cut into 8 contiguous ranges, one per XCD (each has its own
// L2), and a block first drains the range of the XCD it runs on, then helps the others,
// so the CUs finish together however unequal the tiles are (ragged tiles cost less).
// Every block leaves once every counter is past its range.
template <int MODE, int BT>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16(GemmArgs a) {
  // one LDS object (a second one costs a full DMA drain per stage: the compiler's wait
  // insertion then cannot tell the DMA targets from the operand reads); the tile index
  // sits past the stage ring
  constexpr int kRing = NST * (BW + BT) * BK;
  __shared__ __attribute__((aligned(1024))) bf16_t lds[kRing + 64];
  int* next_tile = reinterpret_cast<int*>(lds + kRing);
  const int n_m = MODE == kGemmWgrad ? a.n_m : *a.n_tiles;
  const int n_n = a.n_tiles_n;
  const int G = n_m * n_n * (MODE == kGemmPlainSplit || MODE == kGemmDgradSplit ? a.splits : 1);
  const int per_xcd = (G + 7) / 8;
  // XCC_ID hardware register (bits 3:0): the XCD this block runs on
  int xcd = static_cast<int>(__builtin_amdgcn_s_getreg((3 << 11) | 20)) & 15;
  if (xcd >= 8) xcd = blockIdx.x & 7;
  for (;;) {
    if (threadIdx.x == 0) {
      int L = -1;
      for (int v = 0; v < 8 && L < 0; ++v) {
        const int x = (xcd + v) & 7;
        if (__hip_atomic_load(&a.queue[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= per_xcd) continue;
        const int t = atomicAdd(&a.queue[x], 1);
        if (t < per_xcd && x * per_xcd + t < G) L = x * per_xcd + t;
      }
      *next_tile = L;
    }
    __syncthreads();
    const int L = __builtin_amdgcn_readfirstlane(*next_tile);
    __syncthreads();  // every wave has read next_tile before it is written again
    if (L < 0) return;
    gemm_tile<MODE, BT>(a, lds, L, n_m, n_n);
  }
}

// ---------------------------------------------------------------------------- fp32
// Plain FMA tiles (64 tokens x 64 output columns, 16x16 threads, 4x4 outputs each);
// the fp32 layer is a small-shape path, not a throughput path.
struct GemmArgsF32 {
  const float* in_r;
  const float* in_s;
  const int32_t* sorted_slot;
  const int32_t* tiles;
  const int32_t* n_tiles;
  const float* w0_r;
  const float* w1_r;
  const float* w0_s;
  const float* w1_s;
  float* out_r;
  float* out_s;
  int N_r, K_r, N_s, K_s;
  int E, k, T;
  int m_bound;
};

constexpr int FBM = 64, FBN = 64, FBK = 16;

template <bool GATED>
__global__ __launch_bounds__(256) void grouped_gemm_f32(GemmArgsF32 a) {
  const int m_idx = blockIdx.x % a.m_bound;
  const int n_tile = blockIdx.x / a.m_bound;
  if (m_idx >= *a.n_tiles) return;
  const int g = a.tiles[m_idx * kTileEntries + 0];
  const int row0 = a.tiles[m_idx * kTileEntries + 1];
  const int row1 = a.tiles[m_idx * kTileEntries + 2];
  const bool shared = g >= a.E;
  const int N = shared ? a.N_s : a.N_r;
  const int K = shared ? a.K_s : a.K_r;
  const int n0 = n_tile * FBN;
  if (n0 >= N) return;
  const int gi = shared ? g - a.E : g;
  const float* w0 = (shared ? a.w0_s : a.w0_r) + static_cast<int64_t>(gi) * N * K;
  const float* w1 = GATED ? (shared ? a.w1_s : a.w1_r) + static_cast<int64_t>(gi) * N * K : nullptr;
  const float* in = shared ? a.in_s : a.in_r;

  __shared__ float xs[FBK][FBM + 1];
  __shared__ float ws0[FBK][FBN + 1];
  __shared__ float ws1[FBK][FBN + 1];
  __shared__ int64_t src_row[FBM];
  const int tid = threadIdx.x;
  if (tid < FBM) {
    int row = row0 + tid;
    row = row < row1 ? row : row0;
    int64_t src;
    if (shared)
      src = GATED ? row : static_cast<int64_t>(gi) * a.T + row;
    else
      src = GATED ? a.sorted_slot[row] / a.k : row;
    src_row[tid] = src;
  }
  __syncthreads();
  const int tx = tid & 15, ty = tid >> 4;
  float c0[4][4] = {}, c1[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FBK) {
    for (int i = tid; i < FBM * FBK; i += 256) {
      const int r = i / FBK, kk = i % FBK;
      xs[kk][r] = in[src_row[r] * K + k0 + kk];
      int n = n0 + r;
      n = n < N ? n : N - 1;
      ws0[kk][r] = w0[static_cast<int64_t>(n) * K + k0 + kk];
      if (GATED) ws1[kk][r] = w1[static_cast<int64_t>(n) * K + k0 + kk];
    }
    __syncthreads();
    for (int kk = 0; kk < FBK; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float xv = xs[kk][ty * 4 + i];
          c0[i][j] = fmaf(xv, ws0[kk][tx * 4 + j], c0[i][j]);
          if (GATED) c1[i][j] = fmaf(xv, ws1[kk][tx * 4 + j], c1[i][j]);
        }
    }
    __syncthreads();
  }
  float* out = shared ? a.out_s : a.out_r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + ty * 4 + i;
    if (row >= row1) continue;
    const int64_t orow = shared ? static_cast<int64_t>(gi) * a.T + row : row;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = c0[i][j];
      if (GATED) v = silu_f32(v) * c1[i][j];
      out[orow * N + n] = v;
    }
  }
}

// ------------------------------------------------------------------- tile table
// One block: per-group tile counts, exclusive scan, then the entries.
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int n_shared, int T, int bm,
                                                           int32_t* __restrict__ tiles,
                                                           int32_t* __restrict__ n_tiles,
                                                           int32_t* __restrict__ queues) {
  __shared__ int scan[1024];
  const int e = threadIdx.x;
  if (e < kQueueInts) queues[e] = 0;  // tile counters of the two persistent launches
  int rows = 0, base_row = 0;
  if (e < E) {
    base_row = offsets[e];
    rows = offsets[e + 1] - base_row;
  }
  const int mine = (rows + bm - 1) / bm;
  scan[e] = mine;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = e >= off ? scan[e - off] : 0;
    __syncthreads();
    scan[e] += v;
    __syncthreads();
  }
  const int first = scan[e] - mine;
  for (int i = 0; i < mine; ++i) {
    int32_t* t = tiles + static_cast<int64_t>(first + i) * kTileEntries;
    t[0] = e;
    t[1] = base_row + i * bm;
    t[2] = min(base_row + (i + 1) * bm, base_row + rows);
    t[3] = raster_run(first, mine, i);
  }
  const int routed_tiles = scan[1023];
  const int per_shared = (T + bm - 1) / bm;
  for (int i = e; i < n_shared * per_shared; i += 1024) {
    const int s = i / per_shared, m = i % per_shared;
    int32_t* t = tiles + static_cast<int64_t>(routed_tiles + i) * kTileEntries;
    t[0] = E + s;
    t[1] = m * bm;
    t[2] = min((m + 1) * bm, T);
    t[3] = raster_run(routed_tiles + s * per_shared, per_shared, m);
  }
  if (e == 0) *n_tiles = routed_tiles + n_shared * per_shared;
}

constexpr int kBT = 256;  // token rows per bf16 tile
int tile_rows(const Shape& s) { return s.dtype == MOE_BF16 ? kBT : FBM; }

// Decode-sized batches past the weight-streaming path (experts averaging at most 16 rows, and
// shared experts seeing at most 64 tokens) run the forward launches on tiles of kDecodeBT token
// rows (grouped_mlp_decode.hip): such launches only stream weights, and a 64-row token part
// leaves the LDS to a deeper ring of weight stages (Mixtral-shaped T = 64: step 0.541 -> 0.536
// ms, both launches 1% faster; a 3-stage ring with two blocks per CU was slower, 0.65 ms).
// 0 keeps them on 256-row tiles.
#ifndef MOE_GEMM_FWD_DECODE
#define MOE_GEMM_FWD_DECODE 1
#endif
constexpr int kDecodeBT = 64;
bool use_decode_tiles(const Shape& s) {
  return MOE_GEMM_FWD_DECODE && s.dtype == MOE_BF16 && !use_small_m(s) && s.T * s.k <= 16 * static_cast<int64_t>(s.E) &&
         (s.n_shared == 0 || s.T <= kDecodeBT);
}
// token rows per tile of the forward launches
int fwd_tile_rows(const Shape& s) { return use_decode_tiles(s) ? kDecodeBT : tile_rows(s); }

int64_t m_tile_bound_rows(const Shape& s, int bm) {
  return (s.max_kept + bm - 1) / bm + s.E + static_cast<int64_t>(s.n_shared) * ((s.T + bm - 1) / bm);
}
// m-tiles of the backward's launches (256-row tiles) and of the forward's (the tile table in
// the grouped workspace holds the larger)
int64_t m_tile_bound(const Shape& s) { return m_tile_bound_rows(s, tile_rows(s)); }
int64_t fwd_m_tile_bound(const Shape& s) { return m_tile_bound_rows(s, fwd_tile_rows(s)); }

struct GroupedWs {
  int32_t* tiles;
  int32_t* n_tiles;  // [0]: m-tile count; [16, 16 + kQueueInts): tile counters
  void* h;
  void* hs;
  float* part;  // split-K partials: the small-batch launches, or the split tiled down launch
};

GroupedWs carve(const Shape& s, void* ws) {
  char* p = static_cast<char*>(ws);
  GroupedWs w;
  const int64_t mb = fwd_m_tile_bound(s);
  w.tiles = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<size_t>(mb) * kTileEntries * sizeof(int32_t));
  w.n_tiles = reinterpret_cast<int32_t*>(p);
  p += 256;
  const size_t es = s.dtype == MOE_BF16 ? 2 : 4;
  w.h = p;
  p += align256(static_cast<size_t>(s.max_kept) * s.f * es);
  w.hs = p;
  p += align256(static_cast<size_t>(s.n_shared) * s.T * s.f_s * es);
  w.part = reinterpret_cast<float*>(p);
  return w;
}

}  // namespace

#if defined(MOE_GEMM_DECODE_TU)
// Built a third time with 64-row token tiles and a ring of 7 stages of 32 (grouped_mlp_decode.hip):
// the forward launches (gated, plain, plain split-K) of decode-sized tiled batches, reached
// through launch_gemm_decode with the caller's GemmArgs.
hipError_t launch_gemm_decode(int mode, unsigned grid, const void* args, hipStream_t st) {
  const GemmArgs& a = *static_cast<const GemmArgs*>(args);
  const dim3 gd(grid), bd(kThreads);
  switch (mode) {
    case kGemmGated: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmGated, kDecodeBT>), gd, bd, 0, st, a); break;
    case kGemmPlain: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmPlain, kDecodeBT>), gd, bd, 0, st, a); break;
    case kGemmPlainSplit: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmPlainSplit, kDecodeBT>), gd, bd, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
#elif defined(MOE_GEMM_WIDE_TU)
// Built a second time with K stages of 64 (grouped_mlp_wide.hip): this translation unit
// provides the launches that read weights stored [N][K] (gated, gated with both products
// saved, plain, plain split-K) of those kernels only. `args`
// is the caller's GemmArgs (the same definition, from the same source).
hipError_t launch_gemm_wide(int mode, unsigned grid, const void* args, hipStream_t st) {
  const GemmArgs& a = *static_cast<const GemmArgs*>(args);
  const dim3 gd(grid), bd(kThreads);
  switch (mode) {
    case kGemmGated: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmGated, kBT>), gd, bd, 0, st, a); break;
    case kGemmPlain: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmPlain, kBT>), gd, bd, 0, st, a); break;
    case kGemmPlainSplit: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmPlainSplit, kBT>), gd, bd, 0, st, a); break;
    case kGemmGatedSave: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmGatedSave, kBT>), gd, bd, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
#else
hipError_t launch_gemm_wide(int mode, unsigned grid, const void* args, hipStream_t st);
hipError_t launch_gemm_decode(int mode, unsigned grid, const void* args, hipStream_t st);

// The launches that read weights stored [N][K] use the kernels with K stages of 64 when the
// routed groups average at least kWideMinRows rows (measured on the DeepSeek-shaped,
// Mixtral-shaped and fine-grained layers: step 14.17 -> 13.71, 2.92 -> 2.81 and 0.929 ->
// 0.916 ms, both grouped launches faster). Smaller groups leave the tiles mostly empty and
// the launch bound by its weight stream, which the deeper ring of stages of 32 keeps further
// ahead (Mixtral-shaped T = 64, 16 rows an expert: gated launch 347 against 390 us). 0 keeps
// every launch on this unit's stages of 32.
#ifndef MOE_GEMM_FWD_WIDE
#define MOE_GEMM_FWD_WIDE 1
#endif
namespace {
constexpr int64_t kWideMinRows = 128;
bool use_wide(int64_t T, int k, int E) { return MOE_GEMM_FWD_WIDE && T * k >= kWideMinRows * E; }
// One launch of the persistent grouped GEMM in a mode that reads weights stored [N][K].
hipError_t launch_forward(int mode, int64_t grid, const GemmArgs& a, hipStream_t st, bool wide,
                          bool decode = false) {
  if (decode) return launch_gemm_decode(mode, static_cast<unsigned>(grid), &a, st);
  if (wide) return launch_gemm_wide(mode, static_cast<unsigned>(grid), &a, st);
  const dim3 gd(static_cast<unsigned>(grid)), bd(kThreads);
  switch (mode) {
    case kGemmGated: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmGated, kBT>), gd, bd, 0, st, a); break;
    case kGemmPlain: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmPlain, kBT>), gd, bd, 0, st, a); break;
    case kGemmPlainSplit: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmPlainSplit, kBT>), gd, bd, 0, st, a); break;
    case kGemmGatedSave: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmGatedSave, kBT>), gd, bd, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

float* small_m_partials(const Shape& s, void* ws) { return carve(s, ws).part; }

int large_down_splits(const Shape& s) {
  if (s.dtype != MOE_BF16 || use_small_m(s)) return 1;
  auto halves = [](int K) { return K % 128 == 0; };  // each half a multiple of 64
  if (s.f >= 2 * s.d && halves(s.f) && (s.n_shared == 0 || halves(s.f_s))) return 2;
  return 1;
}

// fp32 partials of a split-K down launch (the small-batch path keeps its own there)
size_t large_split_ws_bytes(const Shape& s) {
  const int sp = large_down_splits(s);
  if (sp <= 1) return 0;
  const int64_t rows_total = s.max_kept + static_cast<int64_t>(s.n_shared) * s.T;
  return align256(static_cast<size_t>(sp) * rows_total * s.d * sizeof(float));
}

size_t grouped_ws_bytes(const Shape& s) {
  const size_t es = s.dtype == MOE_BF16 ? 2 : 4;
  return align256(static_cast<size_t>(fwd_m_tile_bound(s)) * kTileEntries * sizeof(int32_t)) + 256 +
         align256(static_cast<size_t>(s.max_kept) * s.f * es) +
         align256(static_cast<size_t>(s.n_shared) * s.T * s.f_s * es) +
         std::max(small_m_ws_bytes(s), large_split_ws_bytes(s));
}

// compute units of the current device (cached per device)
int cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int64_t gemm_m_tile_bound(const Shape& s) { return m_tile_bound(s); }

hipError_t launch_build_tiles(const Shape& s, const int32_t* offsets, int32_t* tiles, int32_t* n_tiles,
                              int32_t* queues, hipStream_t st) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, st, offsets, s.E, s.n_shared,
                     static_cast<int>(s.T), tile_rows(s), tiles, n_tiles, queues);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmLaunch& L, hipStream_t st) {
  GemmArgs a{};
  a.in_r = static_cast<const bf16_t*>(L.in_r);
  a.in_s = static_cast<const bf16_t*>(L.in_s);
  a.sorted_slot = L.sorted_slot;
  a.tiles = L.tiles;
  a.n_tiles = L.n_tiles;
  a.w0_r = static_cast<const bf16_t*>(L.w0_r);
  a.w1_r = static_cast<const bf16_t*>(L.w1_r);
  a.w0_s = static_cast<const bf16_t*>(L.w0_s);
  a.w1_s = static_cast<const bf16_t*>(L.w1_s);
  a.out_r = static_cast<bf16_t*>(L.out_r);
  a.out_s = static_cast<bf16_t*>(L.out_s);
  a.N_r = L.N_r;
  a.K_r = L.K_r;
  a.N_s = L.N_s;
  a.K_s = L.K_s;
  a.E = L.E;
  a.k = L.k;
  a.T = L.T;
  a.queue = L.queue;
  a.koff = L.koff;
  a.ld_in_r = L.ld_in_r;
  a.ld_w_r = L.ld_w_r;
  a.ld_in_s = L.ld_in_s;
  a.ld_w_s = L.ld_w_s;
  a.in_s_gstride = L.in_s_gstride;
  a.w_s_gstride = L.w_s_gstride;
  a.M_r = L.M_r;
  a.M_s = L.M_s;
  a.part = L.part;
  const bool split = L.mode == kGemmPlainSplit || L.mode == kGemmDgradSplit;
  a.splits = split ? L.splits : 1;
  a.ksw_r = L.ksw_r;
  a.ksw_s = L.ksw_s;
  a.max_kept = L.max_kept;
  a.part_rows = L.max_kept + static_cast<int64_t>(L.n_shared) * L.T;
  const bool gated = L.mode == kGemmGated || L.mode == kGemmGatedSave;
  const int n_max = L.n_shared > 0 && L.N_s > L.N_r ? L.N_s : L.N_r;
  a.n_tiles_n = gated ? (n_max + BW / 2 - 1) / (BW / 2) : (n_max + BW - 1) / BW;
  int64_t mb = L.m_bound;
  if (L.mode == kGemmWgrad) {
    a.mt_r = (L.M_r + kBT - 1) / kBT;
    a.mt_s = L.n_shared > 0 ? (L.M_s + kBT - 1) / kBT : 1;
    a.n_m = L.E * a.mt_r + L.n_shared * (L.n_shared > 0 ? a.mt_s : 0);
    mb = a.n_m;
  }
  const int64_t grid = std::min<int64_t>(cu_count(), static_cast<int64_t>(a.n_tiles_n) * mb * a.splits);
  if (grid <= 0) return hipSuccess;
  const dim3 gd(static_cast<unsigned>(grid)), bd(kThreads);
  switch (L.mode) {
    case kGemmGated:
    case kGemmPlain:
    case kGemmGatedSave:
    case kGemmPlainSplit: return launch_forward(L.mode, grid, a, st, use_wide(L.T, L.k, L.E));
    case kGemmDgradGather: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmDgradGather, kBT>), gd, bd, 0, st, a); break;
    case kGemmWgrad: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmWgrad, kBT>), gd, bd, 0, st, a); break;
    case kGemmDgrad: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmDgrad, kBT>), gd, bd, 0, st, a); break;
    case kGemmDgradSplit: hipLaunchKernelGGL((grouped_gemm_bf16<kGemmDgradSplit, kBT>), gd, bd, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_grouped_mlp(const Shape& s, const void* x, const int32_t* sorted_slot,
                              const int32_t* offsets, const void* wg, const void* wu,
                              const void* wd, const void* swg, const void* swu, const void* swd,
                              void* y_perm, void* y_shared, void* ws, hipStream_t st, const Fp8Scales& fp8,
                              const SmallCombine& comb, const RouteArgs* route) {
  GroupedWs w = carve(s, ws);
  if (use_small_m(s) || (fp8.gate && small_m_fits(s)))
    return launch_grouped_mlp_small(s, x, sorted_slot, offsets, wg, wu, wd, swg, swu, swd, w.h, w.hs,
                                    w.part, y_perm, y_shared, st, fp8, comb, route);
  if (fp8.gate) return hipErrorInvalidValue;  // FP8 weights: weight-streaming path only
  const bool decode = use_decode_tiles(s);
  const int bm = fwd_tile_rows(s);
  const int64_t mb = fwd_m_tile_bound(s);
  int32_t* queues = w.n_tiles + 16;
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, st, offsets, s.E, s.n_shared,
                     static_cast<int>(s.T), bm, w.tiles, w.n_tiles, queues);
  const int f_max = s.n_shared > 0 && s.f_s > s.f ? s.f_s : s.f;
  if (s.dtype == MOE_BF16) {
    GemmArgs a{};
    a.sorted_slot = sorted_slot;
    a.tiles = w.tiles;
    a.n_tiles = w.n_tiles;
    a.E = s.E;
    a.k = s.k;
    a.T = static_cast<int>(s.T);
    // launch 1: h = silu(x Wg) * (x Wu)
    a.in_r = static_cast<const bf16_t*>(x);
    a.in_s = static_cast<const bf16_t*>(x);
    a.w0_r = static_cast<const bf16_t*>(wg);
    a.w1_r = static_cast<const bf16_t*>(wu);
    a.w0_s = static_cast<const bf16_t*>(swg);
    a.w1_s = static_cast<const bf16_t*>(swu);
    a.out_r = static_cast<bf16_t*>(w.h);
    a.out_s = static_cast<bf16_t*>(w.hs);
    a.N_r = s.f;
    a.K_r = s.d;
    a.N_s = s.f_s;
    a.K_s = s.d;
    a.n_tiles_n = static_cast<int>((f_max + BW / 2 - 1) / (BW / 2));
    a.queue = queues;
    // persistent: one block per CU (the LDS ring admits one), never more than the tiles
    const int n_cu = cu_count();
    const int64_t g1 = std::min<int64_t>(n_cu, static_cast<int64_t>(a.n_tiles_n) * mb);
    timing_begin(MOE_KERNEL_GATE_UP, st);
    const bool wide = use_wide(s.T, s.k, s.E);
    hipError_t le = launch_forward(kGemmGated, g1, a, st, wide, decode);
    timing_end(MOE_KERNEL_GATE_UP, st);
    if (le != hipSuccess) return le;
    // launch 2: y = h Wd
    a.sorted_slot = nullptr;
    a.in_r = static_cast<const bf16_t*>(w.h);
    a.in_s = static_cast<const bf16_t*>(w.hs);
    a.w0_r = static_cast<const bf16_t*>(wd);
    a.w1_r = nullptr;
    a.w0_s = static_cast<const bf16_t*>(swd);
    a.w1_s = nullptr;
    a.out_r = static_cast<bf16_t*>(y_perm);
    a.out_s = static_cast<bf16_t*>(y_shared);
    a.N_r = s.d;
    a.K_r = s.f;
    a.N_s = s.d;
    a.K_s = s.f_s;
    a.n_tiles_n = (s.d + BW - 1) / BW;
    a.queue = queues + 8;
    // a long K against a narrow output: split K in two, fp32 partials reduced in split order
    // (or summed by the layer's combine when y_perm is null)
    const int sp = large_down_splits(s);
    a.splits = sp;
    a.part = w.part;
    a.max_kept = s.max_kept;
    a.part_rows = s.max_kept + static_cast<int64_t>(s.n_shared) * s.T;
    const int64_t g2 = std::min<int64_t>(n_cu, static_cast<int64_t>(a.n_tiles_n) * mb * sp);
    timing_begin(MOE_KERNEL_DOWN, st);
    le = launch_forward(sp > 1 ? kGemmPlainSplit : kGemmPlain, g2, a, st, wide, decode);
    timing_end(MOE_KERNEL_DOWN, st);
    if (le != hipSuccess) return le;
    if (sp > 1 && y_perm != nullptr) return launch_split_reduce(s, w.part, sp, offsets, y_perm, y_shared, st);
  } else {
    GemmArgsF32 a{};
    a.sorted_slot = sorted_slot;
    a.tiles = w.tiles;
    a.n_tiles = w.n_tiles;
    a.E = s.E;
    a.k = s.k;
    a.T = static_cast<int>(s.T);
    a.m_bound = static_cast<int>(mb);
    a.in_r = static_cast<const float*>(x);
    a.in_s = static_cast<const float*>(x);
    a.w0_r = static_cast<const float*>(wg);
    a.w1_r = static_cast<const float*>(wu);
    a.w0_s = static_cast<const float*>(swg);
    a.w1_s = static_cast<const float*>(swu);
    a.out_r = static_cast<float*>(w.h);
    a.out_s = static_cast<float*>(w.hs);
    a.N_r = s.f;
    a.K_r = s.d;
    a.N_s = s.f_s;
    a.K_s = s.d;
    const int64_t nt1 = (f_max + FBN - 1) / FBN;
    timing_begin(MOE_KERNEL_GATE_UP, st);
    hipLaunchKernelGGL(grouped_gemm_f32<true>, dim3(static_cast<unsigned>(nt1 * mb)), dim3(256), 0,
                       st, a);
    timing_end(MOE_KERNEL_GATE_UP, st);
    a.sorted_slot = nullptr;
    a.in_r = static_cast<const float*>(w.h);
    a.in_s = static_cast<const float*>(w.hs);
    a.w0_r = static_cast<const float*>(wd);
    a.w1_r = nullptr;
    a.w0_s = static_cast<const float*>(swd);
    a.w1_s = nullptr;
    a.out_r = static_cast<float*>(y_perm);
    a.out_s = static_cast<float*>(y_shared);
    a.N_r = s.d;
    a.K_r = s.f;
    a.N_s = s.d;
    a.K_s = s.f_s;
    const int64_t nt2 = (s.d + FBN - 1) / FBN;
    timing_begin(MOE_KERNEL_DOWN, st);
    hipLaunchKernelGGL(grouped_gemm_f32<false>, dim3(static_cast<unsigned>(nt2 * mb)), dim3(256), 0,
                       st, a);
    timing_end(MOE_KERNEL_DOWN, st);
  }
  return hipGetLastError();
}

#endif  // MOE_GEMM_WIDE_TU

}  // namespace moe

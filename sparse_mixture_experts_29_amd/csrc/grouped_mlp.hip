// Grouped expert MLP: for every expert, its batch of gathered token rows through the
// SwiGLU block (silu(v Wg) * (v Wu)) Wd, as two grouped GEMM launches.
// Pages: klaylearn.com/glossary/mixture-of-experts, definition ("running grouped GEMMs on
// each expert's batch"); techbonafide.com "Mixture of Experts (MoE) Explained", section
// "Experts as Specialized Subnetworks" (an expert is a standard feed-forward block);
// shubhamtatvamasi.com/llm-inference/moe, section "The router" (shared experts every token
// always visits).
//
// Groups: the E routed experts (rows = their slice of the grouped order, input row =
// x[sorted_slot[p] / k]) and the n_s shared experts (rows = all T tokens, identity
// gather). A device-built tile table lists (group, first row, end row) of every BM-row
// tile, so expert sizes never travel to the host and a skewed expert simply owns more
// tiles. Launch 1 (gated) computes h = silu(v Wg) * (v Wu) for a 128-column slice of f,
// with the gate and up rows of that slice side by side in LDS; launch 2 computes
// y = h Wd for a 256-column slice of d.
//
// bf16 tile: 256 threads (4 waves, 2 x 2), 256 weight rows x 128 token rows x BK 64,
// two LDS stages (96 KB) filled from registers prefetched one K step ahead.
// MFMA v_mfma_f32_32x32x16_bf16 with the WEIGHT rows as operand A and the token rows as
// operand B: the accumulator then holds 4 consecutive output columns per lane, stored as
// one 8-byte write. LDS rows are 128 B; 16-byte chunk c of row r lives at chunk
// c ^ (r & 7) ^ ((r >> 3) & 1), which keeps both the row-wise fills and the MFMA
// operand reads (32 rows x one chunk) free of bank conflicts.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 128;   // token rows per tile
constexpr int BNW = 256;  // weight rows per tile
constexpr int BK = 64;    // K per stage
constexpr int kTileEntries = 4;  // int32 per tile-table entry

struct GemmArgs {
  const bf16_t* in_r;        // routed input rows: x [T][K] (gather) or h [rows][K]
  const bf16_t* in_s;        // shared input rows: x [T][K] or hs [n_s*T][K]
  const int32_t* sorted_slot;  // gather for routed rows (gated launch), else nullptr
  const int32_t* tiles;      // [n][4] {group, row_begin, row_end, 0}
  const int32_t* n_tiles;    // device count
  const bf16_t* w0_r;        // routed weights [E][N_r][K_r] (gate, or down)
  const bf16_t* w1_r;        // routed up weights (gated)
  const bf16_t* w0_s;        // shared weights [n_s][N_s][K_s]
  const bf16_t* w1_s;
  bf16_t* out_r;             // [rows][N_r]
  bf16_t* out_s;             // [n_s*T][N_s]
  int N_r, K_r, N_s, K_s;
  int E, k, T;
  int m_bound;               // tile-table capacity (grid's m extent)
};

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <bool GATED>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16(GemmArgs a) {
  const int m_idx = blockIdx.x % a.m_bound;
  const int n_tile = blockIdx.x / a.m_bound;
  if (m_idx >= *a.n_tiles) return;
  const int g = a.tiles[m_idx * kTileEntries + 0];
  const int row0 = a.tiles[m_idx * kTileEntries + 1];
  const int row1 = a.tiles[m_idx * kTileEntries + 2];
  const bool shared = g >= a.E;
  const int N = shared ? a.N_s : a.N_r;
  const int K = shared ? a.K_s : a.K_r;
  constexpr int BNO = GATED ? BNW / 2 : BNW;  // output columns per tile
  const int n0 = n_tile * BNO;
  if (n0 >= N) return;

  const int gi = shared ? g - a.E : g;
  const bf16_t* w0 = (shared ? a.w0_s : a.w0_r) + static_cast<int64_t>(gi) * N * K;
  const bf16_t* w1 = GATED ? (shared ? a.w1_s : a.w1_r) + static_cast<int64_t>(gi) * N * K : nullptr;

  __shared__ __attribute__((aligned(16))) bf16_t lds[2][(BNW + BM) * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ch = tid & 7;   // 16-byte chunk within a 64-wide K row
  const int rq = tid >> 3;  // 0..31: row within a group of 32

  // global row pointers for the fills (fixed over K)
  const bf16_t* wp[BNW / 32];
#pragma unroll
  for (int i = 0; i < BNW / 32; ++i) {
    const int r = rq + 32 * i;
    int n;
    const bf16_t* base;
    if (GATED) {
      base = r < BNW / 2 ? w0 : w1;
      n = n0 + (r < BNW / 2 ? r : r - BNW / 2);
    } else {
      base = w0;
      n = n0 + r;
    }
    n = n < N ? n : N - 1;
    wp[i] = base + static_cast<int64_t>(n) * K + ch * 8;
  }
  const bf16_t* xp[BM / 32];
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) {
    int row = row0 + rq + 32 * i;
    row = row < row1 ? row : row0;
    int64_t src;
    if (shared) {
      src = GATED ? row : static_cast<int64_t>(gi) * a.T + row;
    } else {
      src = GATED ? a.sorted_slot[row] / a.k : row;
    }
    xp[i] = (shared ? a.in_s : a.in_r) + src * K + ch * 8;
  }

  u32x4 wreg[BNW / 32], xreg[BM / 32];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < BNW / 32; ++i) wreg[i] = *reinterpret_cast<const u32x4*>(wp[i] + k0);
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) xreg[i] = *reinterpret_cast<const u32x4*>(xp[i] + k0);
  };
  auto store_lds = [&](int st) {
    bf16_t* wl = lds[st];
    bf16_t* xl = lds[st] + BNW * BK;
#pragma unroll
    for (int i = 0; i < BNW / 32; ++i) {
      const int r = rq + 32 * i;
      *reinterpret_cast<u32x4*>(wl + r * BK + ((ch ^ swz(r)) << 3)) = wreg[i];
    }
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
      const int r = rq + 32 * i;
      *reinterpret_cast<u32x4*>(xl + r * BK + ((ch ^ swz(r)) << 3)) = xreg[i];
    }
  };

  // wave tile: 128 weight rows (gated: 64 gate + 64 up) x 64 token rows
  const int wn = wave & 1, wm = wave >> 1;
  int wrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (GATED)
      wrow[i] = (i < 2 ? 0 : BNW / 2) + wn * 64 + (i & 1) * 32;
    else
      wrow[i] = wn * 128 + i * 32;
  }
  const int xrow0 = wm * 64;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = K / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  const int l32 = lane & 31, khalf = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < KT) load_global((kt + 1) * BK);
    const bf16_t* wl = lds[st];
    const bf16_t* xl = lds[st] + BNW * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + khalf;
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wrow[i] + l32;
        af[i] = *reinterpret_cast<const bf16x8*>(wl + r * BK + ((c ^ swz(r)) << 3));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = xrow0 + j * 32 + l32;
        bfr[j] = *reinterpret_cast<const bf16x8*>(xl + r * BK + ((c ^ swz(r)) << 3));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_lds(st ^ 1);
    __syncthreads();
  }

  // epilogue. acc[i][j] register r of lane l: weight row wrow[i] + 8*(r/4) + 4*(l/32) + r%4,
  // token row xrow0 + 32*j + l%32.
  bf16_t* out = shared ? a.out_s : a.out_r;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = row0 + xrow0 + j * 32 + l32;
    if (row >= row1) continue;
    const int64_t orow = shared ? static_cast<int64_t>(gi) * a.T + row : row;
    bf16_t* op = out + orow * N;
    if (GATED) {
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
              h[u] = gv / (1.0f + __expf(-gv)) * uv;
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
          const int n = n0 + wrow[i] + q * 8 + khalf * 4;
          if (n < N) {
            uint2 pk;
            pk.x = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
            pk.y = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
            *reinterpret_cast<uint2*>(op + n) = pk;
          }
        }
    }
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
      if (GATED) v = v / (1.0f + __expf(-v)) * c1[i][j];
      out[orow * N + n] = v;
    }
  }
}

// ------------------------------------------------------------------- tile table
// One block: per-group tile counts, exclusive scan, then the entries.
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int n_shared, int T, int bm,
                                                           int32_t* __restrict__ tiles,
                                                           int32_t* __restrict__ n_tiles) {
  __shared__ int scan[1024];
  const int e = threadIdx.x;
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
    t[3] = 0;
  }
  const int routed_tiles = scan[1023];
  const int per_shared = (T + bm - 1) / bm;
  for (int i = e; i < n_shared * per_shared; i += 1024) {
    const int s = i / per_shared, m = i % per_shared;
    int32_t* t = tiles + static_cast<int64_t>(routed_tiles + i) * kTileEntries;
    t[0] = E + s;
    t[1] = m * bm;
    t[2] = min((m + 1) * bm, T);
    t[3] = 0;
  }
  if (e == 0) *n_tiles = routed_tiles + n_shared * per_shared;
}

int tile_rows(const Shape& s) { return s.dtype == MOE_BF16 ? BM : FBM; }

int64_t m_tile_bound(const Shape& s) {
  const int bm = tile_rows(s);
  return (s.max_kept + bm - 1) / bm + s.E + static_cast<int64_t>(s.n_shared) * ((s.T + bm - 1) / bm);
}

struct GroupedWs {
  int32_t* tiles;
  int32_t* n_tiles;
  void* h;
  void* hs;
};

GroupedWs carve(const Shape& s, void* ws) {
  char* p = static_cast<char*>(ws);
  GroupedWs w;
  const int64_t mb = m_tile_bound(s);
  w.tiles = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<size_t>(mb) * kTileEntries * sizeof(int32_t));
  w.n_tiles = reinterpret_cast<int32_t*>(p);
  p += 256;
  const size_t es = s.dtype == MOE_BF16 ? 2 : 4;
  w.h = p;
  p += align256(static_cast<size_t>(s.max_kept) * s.f * es);
  w.hs = p;
  return w;
}

}  // namespace

size_t grouped_ws_bytes(const Shape& s) {
  const size_t es = s.dtype == MOE_BF16 ? 2 : 4;
  return align256(static_cast<size_t>(m_tile_bound(s)) * kTileEntries * sizeof(int32_t)) + 256 +
         align256(static_cast<size_t>(s.max_kept) * s.f * es) +
         align256(static_cast<size_t>(s.n_shared) * s.T * s.f_s * es);
}

hipError_t launch_grouped_mlp(const Shape& s, const void* x, const int32_t* sorted_slot,
                              const int32_t* offsets, const void* wg, const void* wu,
                              const void* wd, const void* swg, const void* swu, const void* swd,
                              void* y_perm, void* y_shared, void* ws, hipStream_t st) {
  GroupedWs w = carve(s, ws);
  const int bm = tile_rows(s);
  const int64_t mb = m_tile_bound(s);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, st, offsets, s.E, s.n_shared,
                     static_cast<int>(s.T), bm, w.tiles, w.n_tiles);
  const int f_max = s.n_shared > 0 && s.f_s > s.f ? s.f_s : s.f;
  if (s.dtype == MOE_BF16) {
    GemmArgs a{};
    a.sorted_slot = sorted_slot;
    a.tiles = w.tiles;
    a.n_tiles = w.n_tiles;
    a.E = s.E;
    a.k = s.k;
    a.T = static_cast<int>(s.T);
    a.m_bound = static_cast<int>(mb);
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
    const int64_t nt1 = (f_max + BNW / 2 - 1) / (BNW / 2);
    hipLaunchKernelGGL(grouped_gemm_bf16<true>, dim3(static_cast<unsigned>(nt1 * mb)), dim3(kThreads),
                       0, st, a);
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
    const int64_t nt2 = (s.d + BNW - 1) / BNW;
    hipLaunchKernelGGL(grouped_gemm_bf16<false>, dim3(static_cast<unsigned>(nt2 * mb)), dim3(kThreads),
                       0, st, a);
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
    hipLaunchKernelGGL(grouped_gemm_f32<true>, dim3(static_cast<unsigned>(nt1 * mb)), dim3(256), 0,
                       st, a);
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
    hipLaunchKernelGGL(grouped_gemm_f32<false>, dim3(static_cast<unsigned>(nt2 * mb)), dim3(256), 0,
                       st, a);
  }
  return hipGetLastError();
}

}  // namespace moe

// Router: logits = x . W_r^T + b, top-k per token (ties to the lower expert index), gates
// renormalised over the chosen k (softmax, or sigmoid as in DeepSeek-V3).
// Pages: shubhamtatvamasi.com/llm-inference/moe "Mixture of Experts", section "The router"
// and Q&A "How does a top-k router work?"; shipai.vats.cc "How routing works (intuition)".
//
// E <= 8, or E <= 32 with a small batch: vector-ALU kernel (router_small_e_kernel).
// Larger E: one block of 256 threads owns BT tokens and every expert:
//   1. logits tile [BT][E] accumulated in fp32 (bf16: MFMA 16x16x32, W_r rows as the A
//      operand, token rows as B; fp32: plain FMA) and parked in LDS;
//   2. each wave takes BT/4 tokens and runs k rounds of a wave-wide argmax over the
//      token's E logits (key: larger logit, then lower index), then the gates.
// The bf16 K loop reads 64 contiguous bytes per lane per operand: lane l covers
// k in [32*(l/16), 32*(l/16)+32) of a 128-wide K block and feeds it to 4 MFMAs. The
// MFMA sees a permuted K order, identical for both operands, so the dot products are
// unchanged.
#include "common.h"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;
constexpr int kExpertChunk = 256;  // experts per MFMA pass (4 waves x 64)

template <int BT>
__device__ void topk_and_gates(const float* lg, int ld, int t0, int T, int E, int k, int gating,
                               int32_t* idx, float* gate) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kTokPerWave = BT / 4;
  const int R = (E + 63) / 64;  // candidates per lane
  for (int tt = 0; tt < kTokPerWave; ++tt) {
    const int tl = wave * kTokPerWave + tt;
    const int t = t0 + tl;
    if (t >= T) break;
    const float* row = lg + tl * ld;
    uint32_t taken = 0;  // bit r: candidate lane + 64 r already chosen
    float chosen_l = 0.f;
    int chosen_e = 0;
    float my_l = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      // lane-local best among untaken candidates
      float bl = -INFINITY;
      int be = 0x7fffffff;
      for (int r = 0; r < R; ++r) {
        const int e = lane + 64 * r;
        if (e < E && !((taken >> r) & 1u)) {
          const float v = row[e];
          if (v > bl || (v == bl && e < be)) { bl = v; be = e; }
        }
      }
      // wave argmax: larger logit, then lower index
      for (int off = 32; off >= 1; off >>= 1) {
        const float ol = __shfl_xor(bl, off);
        const int oe = __shfl_xor(be, off);
        if (ol > bl || (ol == bl && oe < be)) { bl = ol; be = oe; }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (lane == j) { my_l = bl; my_e = be; }
      if (j == 0) { chosen_l = bl; chosen_e = be; }
    }
    (void)chosen_e;
    // gates over the k chosen logits held by lanes 0..k-1
    float p = 0.f;
    if (lane < k) {
      p = (gating == MOE_SOFTMAX) ? __expf(my_l - chosen_l) : sigmoid_f32(my_l);
    }
    float sum = p;
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane < k) {
      idx[static_cast<int64_t>(t) * k + lane] = my_e;
      gate[static_cast<int64_t>(t) * k + lane] = p / sum;
    }
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

  for (int e0 = 0; e0 < E; e0 += kExpertChunk) {
    const int ew = e0 + wave * 64;  // this wave's 64 experts
    if (ew < E) {
      const bf16_t* wrow[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        int e = ew + mt * 16 + l16;
        e = e < E ? e : E - 1;
        wrow[mt] = w + static_cast<int64_t>(e) * d;
      }
      f32x4 acc[4][NT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

      int kb = 0;
      for (; kb + 128 <= d; kb += 128) {
        const int ko = kb + quad * 32;
        u32x4 a[4][4], b[NT][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int c = 0; c < 4; ++c) a[mt][c] = *reinterpret_cast<const u32x4*>(wrow[mt] + ko + c * 8);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int c = 0; c < 4; ++c) b[nt][c] = *reinterpret_cast<const u32x4*>(xrow[nt] + ko + c * 8);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, a[mt][c]), __builtin_bit_cast(bf16x8, b[nt][c]),
                  acc[mt][nt], 0, 0, 0);
      }
      if (kb < d) {  // 64-wide tail: lane covers 16 k values
        const int ko = kb + quad * 16;
        u32x4 a[4][2], b[NT][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int c = 0; c < 2; ++c) a[mt][c] = *reinterpret_cast<const u32x4*>(wrow[mt] + ko + c * 8);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int c = 0; c < 2; ++c) b[nt][c] = *reinterpret_cast<const u32x4*>(xrow[nt] + ko + c * 8);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, a[mt][c]), __builtin_bit_cast(bf16x8, b[nt][c]),
                  acc[mt][nt], 0, 0, 0);
      }
      // C layout (16x16): lane holds rows (experts) 4*quad + i, column (token) l16
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = ew + mt * 16 + quad * 4 + i;
            if (e < E) lg[(nt * 16 + l16) * ld + e] = acc[mt][nt][i] + (bias ? bias[e] : 0.f);
          }
    }
  }
  __syncthreads();
  if (logits) {
    for (int i = threadIdx.x; i < BT * E; i += kRouterThreads) {
      const int tl = i / E, e = i - tl * E;
      if (t0 + tl < T) logits[static_cast<int64_t>(t0 + tl) * E + e] = lg[tl * ld + e];
    }
  }
  topk_and_gates<BT>(lg, ld, t0, T, E, k, gating, idx, gate);
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
  topk_and_gates<BT>(lg, ld, t0, T, E, k, gating, idx, gate);
}

// Small expert counts (E <= 32): a block of 256 threads owns TB tokens and splits d over all
// its lanes (8 consecutive elements per lane per pass), so even one token keeps 256 lanes'
// loads in flight. Every load is issued unconditionally (rows past the end are clamped to
// the last one and ignored), which keeps the compiler's count of loads in flight exact.
// Partial sums (TB * EMAX = 32 per lane) are summed through LDS in a fixed order: each
// thread folds one value over 32 lanes, then each logit over the 8 groups of lanes; wave w
// then runs top-k and the gates for token w.
template <typename T, int EMAX, int TB>
__global__ __launch_bounds__(256) void router_small_e_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const float* __restrict__ bias,
    int32_t* __restrict__ idx, float* __restrict__ gate, float* __restrict__ logits, int n_tok,
    int d, int E, int k, int gating) {
  static_assert(TB * EMAX == 32, "32 partial sums per lane");
  __shared__ float part[256][33];  // +1: rows fall on distinct banks
  __shared__ float red[8][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TB;
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
  // d is a multiple of 64, so a lane's 8 elements never straddle the end
  for (int c = threadIdx.x * 8; c < d; c += 2048) {
    u32x4 xr_raw[TB][kVec], wr_raw[EMAX][kVec];
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int q = 0; q < kVec; ++q) xr_raw[b][q] = *reinterpret_cast<const u32x4*>(xr[b] + c + 4 * q);
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
#pragma unroll
      for (int q = 0; q < kVec; ++q) wr_raw[e][q] = *reinterpret_cast<const u32x4*>(wr[e] + c + 4 * q);
    float xv[TB][8];
#pragma unroll
    for (int b = 0; b < TB; ++b) widen(xr_raw[b], xv[b]);
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      float wv[8];
      widen(wr_raw[e], wv);
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[b * EMAX + e] = fmaf(xv[b][i], wv[i], acc[b * EMAX + e]);
    }
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) part[threadIdx.x][i] = acc[i];
  __syncthreads();
  {
    const int o = threadIdx.x & 31, grp = threadIdx.x >> 5;
    float sum = 0.f;
    for (int l = 0; l < 32; ++l) sum += part[grp * 32 + l][o];
    red[grp][o] = sum;
  }
  __syncthreads();
  const int t = t0 + wave;
  if (wave >= TB || t >= n_tok) return;
  float my = -INFINITY;
  if (lane < E) {
    const int j = wave * EMAX + lane;
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) sum += red[g][j];
    my = sum + (bias ? bias[lane] : 0.f);
  }
  if (logits && lane < E) logits[static_cast<int64_t>(t) * E + lane] = my;
  // top-k: k rounds of a wave argmax (larger logit, then lower index)
  bool taken = false;
  float first = 0.f, mine_l = 0.f;
  int mine_e = 0;
  for (int j = 0; j < k; ++j) {
    float bl = (lane < E && !taken) ? my : -INFINITY;
    int be = (lane < E && !taken) ? lane : 0x7fffffff;
    for (int off = 32; off >= 1; off >>= 1) {
      const float ol = __shfl_xor(bl, off);
      const int oe = __shfl_xor(be, off);
      if (ol > bl || (ol == bl && oe < be)) { bl = ol; be = oe; }
    }
    if (lane == be) taken = true;
    if (lane == j) { mine_l = bl; mine_e = be; }
    if (j == 0) first = bl;
  }
  float p = 0.f;
  if (lane < k) p = (gating == MOE_SOFTMAX) ? __expf(mine_l - first) : sigmoid_f32(mine_l);
  float sum = p;
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    idx[static_cast<int64_t>(t) * k + lane] = mine_e;
    gate[static_cast<int64_t>(t) * k + lane] = p / sum;
  }
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
  const bool small_e = s.E <= 256;
  const int BT = small_e ? 64 : 16;
  const size_t lds = static_cast<size_t>(BT) * (s.E + 4) * sizeof(float);
  const dim3 grid((T + BT - 1) / BT), block(kRouterThreads);
  timing_begin(MOE_KERNEL_ROUTER, st);
  if (s.dtype == MOE_BF16) {
    auto kern = small_e ? router_bf16_kernel<64> : router_bf16_kernel<16>;
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(lds));
    hipLaunchKernelGGL(kern, grid, block, lds, st, static_cast<const bf16_t*>(x),
                       static_cast<const bf16_t*>(w_router), bias, idx, gate, logits, T, s.d, s.E,
                       s.k, s.gating);
  } else {
    auto kern = small_e ? router_f32_kernel<64> : router_f32_kernel<16>;
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(lds));
    hipLaunchKernelGGL(kern, grid, block, lds, st, static_cast<const float*>(x),
                       static_cast<const float*>(w_router), bias, idx, gate, logits, T, s.d, s.E,
                       s.k, s.gating);
  }
  timing_end(MOE_KERNEL_ROUTER, st);
  return hipGetLastError();
}

}  // namespace moe

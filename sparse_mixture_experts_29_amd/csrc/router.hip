// Router: logits = x . W_r^T + b, top-k per token (ties to the lower expert index), gates
// renormalised over the chosen k (softmax, or sigmoid as in DeepSeek-V3).
// Pages: shubhamtatvamasi.com/llm-inference/moe "Mixture of Experts", section "The router"
// and Q&A "How does a top-k router work?"; shipai.vats.cc "How routing works (intuition)".
//
// One block of 256 threads owns BT tokens and every expert:
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

}  // namespace

hipError_t launch_route(const Shape& s, const void* x, const void* w_router, const float* bias,
                        int32_t* idx, float* gate, float* logits, hipStream_t st) {
  const int T = static_cast<int>(s.T);
  const bool small_e = s.E <= 256;
  const int BT = small_e ? 64 : 16;
  const size_t lds = static_cast<size_t>(BT) * (s.E + 4) * sizeof(float);
  const dim3 grid((T + BT - 1) / BT), block(kRouterThreads);
  timing_begin(MOE_KERNEL_ROUTER, st);
  if (s.dtype == MOE_BF16) {
    auto kern = small_e ? router_bf16_kernel<64> : router_bf16_kernel<16>;
    hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                        static_cast<int>(lds));
    hipLaunchKernelGGL(kern, grid, block, lds, st, static_cast<const bf16_t*>(x),
                       static_cast<const bf16_t*>(w_router), bias, idx, gate, logits, T, s.d, s.E,
                       s.k, s.gating);
  } else {
    auto kern = small_e ? router_f32_kernel<64> : router_f32_kernel<16>;
    hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                        static_cast<int>(lds));
    hipLaunchKernelGGL(kern, grid, block, lds, st, static_cast<const float*>(x),
                       static_cast<const float*>(w_router), bias, idx, gate, logits, T, s.d, s.E,
                       s.k, s.gating);
  }
  timing_end(MOE_KERNEL_ROUTER, st);
  return hipGetLastError();
}

}  // namespace moe

// Backward pass of the MoE layer: the element-wise, transpose and router kernels around the
// grouped GEMM launches (grouped_mlp.hip) that moe_layer_backward chains.
// Pages: techbonafide.com "Mixture of Experts (MoE) Explained" and klaylearn.com (MoE shapes
// training as well as inference; mature implementations add auxiliary balancing losses, as
// in the Switch Transformer work); shipai.vats.cc "Mixture of Experts (MoE)" (training adds
// load-balancing losses); shubhamtatvamasi.com/llm-inference/moe, "The router" and "Load
// imbalance" (the forward being differentiated).
//
// With the forward a = v Wg^T, b = v Wu^T, h = silu(a) b, y_p = h Wd^T, y_t = sum_j g_j y_p:
//   u = dy_t Wd (the down dgrad of the unscaled output gradient, a grouped GEMM),
//   dg_j = dy_t . y_p = u . h,  dh = g_j u,  da = dh b silu'(a),  db = dh silu(a)
// (swiglu_bwd_kernel); the gate, up and down weight gradients are grouped GEMMs over
// transposed, zero-padded per-expert segments of the activations (transpose_segments_kernel);
// the router gradient follows the softmax or sigmoid renormalisation of the chosen gates,
// plus the load-balancing loss aux_coef * E * sum_e f_e P_e (router_bwd_kernel).
#include "common.h"

namespace moe {
namespace {

constexpr int kTile = 64;  // transpose tile of the activation segments (rows x columns)

// poff[e] = sum over e' < e of kept rows of e' rounded up to 64 (one block, E <= 1024).
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int32_t* __restrict__ poff) {
  __shared__ int scan[1024];
  const int e = threadIdx.x;
  const int n = e < E ? offsets[e + 1] - offsets[e] : 0;
  const int mine = (n + kTile - 1) / kTile * kTile;
  scan[e] = mine;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = e >= off ? scan[e - off] : 0;
    __syncthreads();
    scan[e] += v;
    __syncthreads();
  }
  if (e < E) poff[e + 1] = scan[e];
  if (e == 0) poff[0] = 0;
}

// Transposed, zero-padded segments: for segment g (rows [off[g], off[g+1]) of the source
// in grouped order) and column c < C,
//   dst[c][poff[g] + i] = scale * src[row(i)][c]  for i < len, 0 for len <= i < pad64(len)
// with row(i) = sorted_slot[off[g] + i] / k (gather) or off[g] + i, and scale = the gate of
// that pair (gate != null) or 1. With off == null there is one segment of `len1` rows
// starting at row 0 (the shared experts' token rows), repeated over blockIdx.z batches.
// Blocks: x = 64-column tiles, y = 64-row tiles of the padded space, z = batch.
__global__ __launch_bounds__(256) void transpose_segments_kernel(
    const bf16_t* __restrict__ src, int src_ld, int64_t src_bstride, const int32_t* __restrict__ off,
    const int32_t* __restrict__ poff, int nseg, int len1, const int32_t* __restrict__ sorted_slot, int k,
    const float* __restrict__ gate, int C, bf16_t* __restrict__ dst, int ldd, int64_t dst_bstride) {
  __shared__ bf16_t tile[kTile][kTile + 2];
  const int p0 = blockIdx.y * kTile;
  int seg_p, seg_row, len;
  if (off != nullptr) {
    if (p0 >= poff[nseg]) return;
    int lo = 0, hi = nseg - 1;  // last g with poff[g] <= p0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (poff[mid] <= p0) lo = mid;
      else hi = mid - 1;
    }
    seg_p = poff[lo];
    seg_row = off[lo];
    len = off[lo + 1] - seg_row;
  } else {
    seg_p = 0;
    seg_row = 0;
    len = len1;
  }
  const int c0 = blockIdx.x * kTile;
  const bf16_t* s = src + blockIdx.z * src_bstride;
  bf16_t* d = dst + blockIdx.z * dst_bstride;
  const int t = threadIdx.x;
  {
    const int r = t >> 2, cq = (t & 3) * 16;
    const int i = p0 - seg_p + r;
    uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (i < len) {
      int64_t row = seg_row + i;
      float sc = 1.f;
      if (sorted_slot != nullptr) {
        const int slot = sorted_slot[seg_row + i];
        row = slot / k;
        if (gate != nullptr) sc = gate[slot];
      }
      const uint4* p = reinterpret_cast<const uint4*>(s + row * src_ld + c0 + cq);
      const uint4 v0 = p[0], v1 = p[1];
      const uint32_t raw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (gate != nullptr)
          w[q] = pack_bf16x2(bf16_to_f32(static_cast<bf16_t>(raw[q] & 0xFFFF)) * sc,
                             bf16_to_f32(static_cast<bf16_t>(raw[q] >> 16)) * sc);
        else
          w[q] = raw[q];
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      tile[r][cq + 2 * q] = static_cast<bf16_t>(w[q] & 0xFFFF);
      tile[r][cq + 2 * q + 1] = static_cast<bf16_t>(w[q] >> 16);
    }
  }
  __syncthreads();
  {
    const int c = t >> 2, rq = (t & 3) * 16;
    if (c0 + c >= C) return;
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      w[q] = static_cast<uint32_t>(tile[rq + 2 * q][c]) | (static_cast<uint32_t>(tile[rq + 2 * q + 1][c]) << 16);
    uint4* p = reinterpret_cast<uint4*>(d + static_cast<int64_t>(c0 + c) * ldd + p0 + rq);
    p[0] = make_uint4(w[0], w[1], w[2], w[3]);
    p[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// SwiGLU backward, one wave per row. Routed rows p < N_kept (ab, u, dab, h: [max_kept][.]):
// g = gate of the pair, dg written to d_gate[slot]; shared rows q < n_s*T (ab_s ...): g = 1.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(
    const bf16_t* __restrict__ ab, const bf16_t* __restrict__ u, const bf16_t* __restrict__ ab_s,
    const bf16_t* __restrict__ u_s, const int32_t* __restrict__ offsets, int E,
    const int32_t* __restrict__ sorted_slot, const float* __restrict__ gate, int64_t max_kept, int64_t shared_rows,
    int f, int f_s, bf16_t* __restrict__ dab, bf16_t* __restrict__ h, bf16_t* __restrict__ dab_s,
    bf16_t* __restrict__ hs, float* __restrict__ d_gate) {
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const bool routed = w < max_kept;
  int64_t row;
  int F;
  float g = 1.f;
  int slot = -1;
  const bf16_t *pa, *pu;
  bf16_t *pd, *ph;
  if (routed) {
    if (w >= offsets[E]) return;
    row = w;
    F = f;
    slot = sorted_slot[w];
    g = gate[slot];
    pa = ab + row * 2 * F;
    pu = u + row * F;
    pd = dab + row * 2 * F;
    ph = h + row * F;
  } else {
    row = w - max_kept;
    if (row >= shared_rows) return;
    F = f_s;
    pa = ab_s + row * 2 * F;
    pu = u_s + row * F;
    pd = dab_s + row * 2 * F;
    ph = hs + row * F;
  }
  float dot = 0.f;
  for (int c = lane * 8; c < F; c += 8 * kWave) {
    const uint4 va = *reinterpret_cast<const uint4*>(pa + c);
    const uint4 vb = *reinterpret_cast<const uint4*>(pa + F + c);
    const uint4 vu = *reinterpret_cast<const uint4*>(pu + c);
    const uint32_t A[4] = {va.x, va.y, va.z, va.w}, B[4] = {vb.x, vb.y, vb.z, vb.w}, U[4] = {vu.x, vu.y, vu.z, vu.w};
    uint32_t DA[4], DB[4], H[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float da2[2], db2[2], h2[2];
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const float a = bf16_to_f32(static_cast<bf16_t>(z ? A[q] >> 16 : A[q] & 0xFFFF));
        const float b = bf16_to_f32(static_cast<bf16_t>(z ? B[q] >> 16 : B[q] & 0xFFFF));
        const float uu = bf16_to_f32(static_cast<bf16_t>(z ? U[q] >> 16 : U[q] & 0xFFFF));
        const float s = sigmoid_f32(a);
        const float sa = a * s;  // silu(a)
        const float hv = sa * b;
        dot += uu * hv;
        const float dh = g * uu;
        da2[z] = dh * b * (s + sa * (1.f - s));
        db2[z] = dh * sa;
        h2[z] = hv;
      }
      DA[q] = pack_bf16x2(da2[0], da2[1]);
      DB[q] = pack_bf16x2(db2[0], db2[1]);
      H[q] = pack_bf16x2(h2[0], h2[1]);
    }
    *reinterpret_cast<uint4*>(pd + c) = make_uint4(DA[0], DA[1], DA[2], DA[3]);
    *reinterpret_cast<uint4*>(pd + F + c) = make_uint4(DB[0], DB[1], DB[2], DB[3]);
    *reinterpret_cast<uint4*>(ph + c) = make_uint4(H[0], H[1], H[2], H[3]);
  }
  if (routed) {
    dot = wave_sum(dot);
    if (lane == 0) d_gate[slot] = dot;
  }
}

constexpr int kMaxEPerLane = 16;  // E <= 1024 over a 64-lane wave

// Router backward, one wave per token: dl[t][e] for every expert (fp32) from the gate
// gradients of the chosen experts and, with aux_coef != 0, the load-balancing loss; aux_part[t]
// = (aux_coef E / T) sum_e f_e p[t][e], the token's share of that loss.
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ logits, const int32_t* __restrict__ idx,
                                                         const float* __restrict__ gate,
                                                         const float* __restrict__ d_gate,
                                                         const int32_t* __restrict__ counts, int64_t T, int E, int k,
                                                         int gating, float aux_coef, float* __restrict__ dl,
                                                         float* __restrict__ aux_part) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const float* lt = logits + t * E;
  // chosen experts: lane j < k holds pair j
  int ej = -1;
  float gj = 0.f, dgj = 0.f, lj = 0.f;
  if (lane < k) {
    ej = idx[t * k + lane];
    gj = gate[t * k + lane];
    dgj = d_gate[t * k + lane];
    lj = lt[ej];
  }
  const float inner = wave_sum(gj * dgj);
  float dsel;
  if (gating == MOE_SOFTMAX) {
    dsel = gj * (dgj - inner);
  } else {
    const float s = lane < k ? sigmoid_f32(lj) : 0.f;
    const float S = wave_sum(s);
    dsel = (dgj - inner) / S * s * (1.f - s);
  }
  float acc[kMaxEPerLane];
#pragma unroll
  for (int m = 0; m < kMaxEPerLane; ++m) acc[m] = 0.f;
  if (aux_coef != 0.f) {
    const float c = aux_coef * static_cast<float>(E) / static_cast<float>(T);
    const float inv_tk = 1.f / static_cast<float>(T * k);
    float z[kMaxEPerLane], mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < kMaxEPerLane; ++m) {
      const int e = lane + m * kWave;
      z[m] = e < E ? lt[e] : -INFINITY;
      mx = fmaxf(mx, z[m]);
    }
    float Z = 0.f;
    if (gating == MOE_SOFTMAX) {
      mx = wave_max(mx);
#pragma unroll
      for (int m = 0; m < kMaxEPerLane; ++m) {
        z[m] = lane + m * kWave < E ? __expf(z[m] - mx) : 0.f;
        Z += z[m];
      }
    } else {
#pragma unroll
      for (int m = 0; m < kMaxEPerLane; ++m) {
        z[m] = lane + m * kWave < E ? sigmoid_f32(z[m]) : 0.f;
        Z += z[m];
      }
    }
    Z = wave_sum(Z);
    float Fp = 0.f;
#pragma unroll
    for (int m = 0; m < kMaxEPerLane; ++m) {
      const int e = lane + m * kWave;
      if (e < E) Fp += static_cast<float>(counts[e]) * inv_tk * z[m];
    }
    const float F = wave_sum(Fp) / Z;  // sum_e f_e p_e
#pragma unroll
    for (int m = 0; m < kMaxEPerLane; ++m) {
      const int e = lane + m * kWave;
      if (e < E) {
        const float fe = static_cast<float>(counts[e]) * inv_tk;
        const float p = z[m] / Z;
        acc[m] = gating == MOE_SOFTMAX ? c * p * (fe - F) : c * (fe - F) * z[m] * (1.f - z[m]) / Z;
      }
    }
    if (lane == 0) aux_part[t] = c * F;
  } else if (lane == 0) {
    aux_part[t] = 0.f;
  }
  // add the chosen experts' terms to the lanes that own them
  for (int j = 0; j < k; ++j) {
    const int e = __shfl(ej, j, kWave);
    const float v = __shfl(dsel, j, kWave);
#pragma unroll
    for (int m = 0; m < kMaxEPerLane; ++m)
      if (lane + m * kWave == e) acc[m] += v;
  }
  float* dt = dl + t * E;
#pragma unroll
  for (int m = 0; m < kMaxEPerLane; ++m)
    if (lane + m * kWave < E) dt[lane + m * kWave] = acc[m];
}

// out[0] = sum of v[0..n) in a fixed order (one block).
__global__ __launch_bounds__(256) void sum_kernel(const float* __restrict__ v, int64_t n, float* __restrict__ out) {
  __shared__ float red[256];
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += v[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = red[0];
}

// out[e] = sum over t of m[t][e]: one block per e, thread i sums the rows t = i mod 256 in
// ascending order, then a fixed tree over the 256 partial sums.
__global__ __launch_bounds__(256) void col_sum_kernel(const float* __restrict__ m, int64_t T, int E,
                                                      float* __restrict__ out) {
  __shared__ float red[256];
  const int e = blockIdx.x;
  float s = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += 256) s += m[t * E + e];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[e] = red[0];
}

// C[m][n] = sum_k A(m, k) B(k, n), A(m, k) = A[m*sam + k*sak] (fp32), B(k, n) = B[k*ldb + n]
// (bf16). 64 x 64 tiles, 16 x 16 threads of 4 x 4 outputs, K in chunks of 16 through LDS.
// Block z covers k in [z*kc, (z+1)*kc): with one split the result is rounded once to bf16
// into C; with several, each writes its fp32 partial P[z][m][n] and reduce_splits_kernel
// sums them in split order. For the router's weight and input gradients.
__global__ __launch_bounds__(256) void fma_gemm_kernel(const float* __restrict__ A, int64_t sam, int64_t sak,
                                                       const bf16_t* __restrict__ B, int64_t ldb, int64_t M, int N,
                                                       int64_t K, int64_t kc, bf16_t* __restrict__ C, int64_t ldc,
                                                       float* __restrict__ P) {
  __shared__ float As[16][65], Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int n0 = blockIdx.x * 64;
  const int64_t kb = static_cast<int64_t>(blockIdx.z) * kc;
  const int64_t ke = kb + kc < K ? kb + kc : K;
  float c[4][4] = {};
  for (int64_t k0 = kb; k0 < ke; k0 += 16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = threadIdx.x + q * 256;  // 1024 = 16 x 64
      const int kk = i >> 6, mm = i & 63;
      const int64_t gm = m0 + mm, gk = k0 + kk;
      As[kk][mm] = gm < M && gk < ke ? A[gm * sam + gk * sak] : 0.f;
      const int gn = n0 + mm;
      Bs[kk][mm] = gn < N && gk < ke ? bf16_to_f32(B[gk * ldb + gn]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = As[kk][ty * 4 + q];
        b[q] = Bs[kk][tx * 4 + q];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) c[i][j] = fmaf(a[i], b[j], c[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn >= N) continue;
      if (P != nullptr)
        P[(static_cast<int64_t>(blockIdx.z) * M + gm) * N + gn] = c[i][j];
      else
        C[gm * ldc + gn] = f32_to_bf16(c[i][j]);
    }
  }
}

// C[m][n] = bf16(sum over z < splits of P[z][m][n]), z ascending.
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ P, int splits, int64_t M,
                                                            int N, bf16_t* __restrict__ C, int64_t ldc) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= M * N) return;
  float s = 0.f;
  for (int z = 0; z < splits; ++z) s += P[z * M * N + i];
  C[(i / N) * ldc + i % N] = f32_to_bf16(s);
}

__global__ __launch_bounds__(256) void fill_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

unsigned blocks(int64_t n, int per) { return static_cast<unsigned>((n + per - 1) / per); }

}  // namespace

hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* poff, hipStream_t st) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(1024), 0, st, offsets, E, poff);
  return hipGetLastError();
}

hipError_t launch_transpose_segments(const void* src, int src_ld, int64_t src_bstride, const int32_t* off,
                                     const int32_t* poff, int nseg, int len1, int64_t padded_rows_bound,
                                     const int32_t* sorted_slot, int k, const float* gate, int C, void* dst, int ldd,
                                     int64_t dst_bstride, int batch, hipStream_t st) {
  if (batch <= 0 || padded_rows_bound <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_segments_kernel, dim3(C / kTile, blocks(padded_rows_bound, kTile), batch), dim3(256),
                     0, st, static_cast<const bf16_t*>(src), src_ld, src_bstride, off, poff, nseg, len1, sorted_slot,
                     k, gate, C, static_cast<bf16_t*>(dst), ldd, dst_bstride);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const Shape& s, const void* ab, const void* u, const void* ab_s, const void* u_s,
                             const int32_t* offsets, const int32_t* sorted_slot, const float* gate, void* dab, void* h,
                             void* dab_s, void* hs, float* d_gate, hipStream_t st) {
  const int64_t shared_rows = static_cast<int64_t>(s.n_shared) * s.T;
  const int64_t rows = s.max_kept + shared_rows;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(blocks(rows, 4)), dim3(256), 0, st, static_cast<const bf16_t*>(ab),
                     static_cast<const bf16_t*>(u), static_cast<const bf16_t*>(ab_s), static_cast<const bf16_t*>(u_s),
                     offsets, s.E, sorted_slot, gate, s.max_kept, shared_rows, s.f, s.f_s, static_cast<bf16_t*>(dab),
                     static_cast<bf16_t*>(h), static_cast<bf16_t*>(dab_s), static_cast<bf16_t*>(hs), d_gate);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const Shape& s, const float* logits, const int32_t* idx, const float* gate,
                             const float* d_gate, const int32_t* counts, float aux_coef, float* dl, float* aux_part,
                             float* aux_loss, float* d_bias, hipStream_t st) {
  hipLaunchKernelGGL(router_bwd_kernel, dim3(blocks(s.T, 4)), dim3(256), 0, st, logits, idx, gate, d_gate, counts,
                     s.T, s.E, s.k, s.gating, aux_coef, dl, aux_part);
  if (aux_loss != nullptr) hipLaunchKernelGGL(sum_kernel, dim3(1), dim3(256), 0, st, aux_part, s.T, aux_loss);
  if (d_bias != nullptr) hipLaunchKernelGGL(col_sum_kernel, dim3(s.E), dim3(256), 0, st, dl, s.T, s.E, d_bias);
  return hipGetLastError();
}

int fma_gemm_splits(int64_t M, int N, int64_t K) {
  const int64_t tiles = ((M + 63) / 64) * ((N + 63) / 64);
  int64_t sp = (1024 + tiles - 1) / tiles;      // about 1024 blocks in all
  sp = std::min<int64_t>(sp, (K + 255) / 256);  // each split keeps >= 256 of K
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(sp, 32)));
}

size_t fma_gemm_ws_bytes(int64_t M, int N, int64_t K) {
  const int sp = fma_gemm_splits(M, N, K);
  return sp > 1 ? static_cast<size_t>(sp) * M * N * sizeof(float) : 0;
}

hipError_t launch_fma_gemm(const float* A, int64_t sam, int64_t sak, const void* B, int64_t ldb, int64_t M, int N,
                           int64_t K, void* C, int64_t ldc, float* partials, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int sp = fma_gemm_splits(M, N, K);
  const int64_t kc = ((K + sp - 1) / sp + 15) / 16 * 16;
  float* P = sp > 1 ? partials : nullptr;
  hipLaunchKernelGGL(fma_gemm_kernel, dim3(blocks(N, 64), blocks(M, 64), sp), dim3(256), 0, st, A, sam, sak,
                     static_cast<const bf16_t*>(B), ldb, M, N, K, kc, static_cast<bf16_t*>(C), ldc, P);
  if (sp > 1)
    hipLaunchKernelGGL(reduce_splits_kernel, dim3(blocks(M * N, 256)), dim3(256), 0, st, P, sp, M, N,
                       static_cast<bf16_t*>(C), ldc);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* p, int64_t n, uint32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(blocks(n, 256)), dim3(256), 0, st, static_cast<uint32_t*>(p), n, v);
  return hipGetLastError();
}

}  // namespace moe

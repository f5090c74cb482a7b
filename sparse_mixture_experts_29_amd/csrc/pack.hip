// One-time pack of expert and router weights from the row-vector layout of y = x . W (the
// d x f matrices as the problem statement writes them) into the library's layout, whose rows
// are the output features: every matrix is transposed, batch by batch.
// Pages: shubhamtatvamasi.com/llm-inference/moe, section "The router" (a linear layer scores
// every expert); klaylearn.com/glossary/mixture-of-experts, definition (each expert is a
// feed-forward block run as a grouped GEMM over its batch); techbonafide.com "Mixture of
// Experts (MoE) Explained", section "Experts as Specialized Subnetworks".
//
// A block moves one 64 x 64 tile through LDS (rows padded by one element, so the column
// reads of the transposed write hit distinct banks); ragged edges are masked. Memory-bound
// and run once per set of weights, not per layer call.
#include "common.h"

namespace moe {
namespace {

constexpr int kTile = 64;

// dst[b][c][r] = src[b][r][c] for a batch of R x C matrices (element type T)
template <typename T>
__global__ __launch_bounds__(256) void transpose_batched_kernel(const T* __restrict__ src, T* __restrict__ dst, int R,
                                                                int C) {
  __shared__ T tile[kTile][kTile + 1];
  const int64_t mat = static_cast<int64_t>(R) * C;
  const T* s = src + blockIdx.z * mat;
  T* d = dst + blockIdx.z * mat;
  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  const int tx = threadIdx.x & (kTile - 1), ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kTile; i += 4) {
    const int r = r0 + ty + i, c = c0 + tx;
    if (r < R && c < C) tile[ty + i][tx] = s[static_cast<int64_t>(r) * C + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kTile; i += 4) {
    const int c = c0 + ty + i, r = r0 + tx;
    if (r < R && c < C) d[static_cast<int64_t>(c) * R + r] = tile[tx][ty + i];
  }
}

}  // namespace

hipError_t launch_transpose_batched(const void* src, void* dst, int64_t batch, int R, int C, int elem_bytes,
                                    hipStream_t st) {
  if (batch <= 0 || R <= 0 || C <= 0) return hipSuccess;
  const dim3 grid((C + kTile - 1) / kTile, (R + kTile - 1) / kTile, static_cast<unsigned>(batch));
  if (elem_bytes == 2)
    hipLaunchKernelGGL(transpose_batched_kernel<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(src),
                       static_cast<uint16_t*>(dst), R, C);
  else
    hipLaunchKernelGGL(transpose_batched_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(src),
                       static_cast<float*>(dst), R, C);
  return hipGetLastError();
}

}  // namespace moe

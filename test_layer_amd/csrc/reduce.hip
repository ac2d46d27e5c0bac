// Deterministic reduction of the per-chunk gradient partials and the fast-
// weight update.
//
// The gradient of the inner loss is a sum over token chunks (Eq. 5 of the
// paper-graph summary "VGG-T3: Offline Feed-Forward 3D Reconstruction at
// Scale", section 3.4 "Large-Scale Inference Strategies"); after all chunks
// are summed, one plain gradient-descent update theta <- theta - lr * g is
// applied to all three matrices at once. Each thread owns one parameter and
// adds its P partials (P a power of two) with a fixed pairwise tree, so the
// result is bitwise reproducible and independent of the launch shape.
#include "common.hpp"
#include "kernels.hpp"

namespace vggt3 {
namespace {

template <int P>
__device__ __forceinline__ float tree_sum(const float* __restrict__ src, int64_t stride) {
  float v[P];
#pragma unroll
  for (int p = 0; p < P; ++p) v[p] = src[p * stride];
#pragma unroll
  for (int s = 1; s < P; s *= 2) {
#pragma unroll
    for (int p = 0; p + s < P; p += 2 * s) v[p] = v[p] + v[p + s];
  }
  return v[0];
}

template <int P>
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ part,
                                                      const float* __restrict__ loss_part, int n_heads,
                                                      int per_head, int mode, float* __restrict__ dst,
                                                      float lr, float* __restrict__ loss_out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)n_heads * per_head;
  if (idx < total) {
    const int64_t h = idx / per_head, i = idx % per_head;
    const float g = tree_sum<P>(part + h * P * per_head + i, per_head);
    if (mode == kApply) dst[idx] = dst[idx] - lr * g;
    else if (mode == kStore) dst[idx] = g;
    else dst[idx] = dst[idx] + g;
  }
  if (loss_out != nullptr && idx < n_heads) {
    const float L = tree_sum<P>(loss_part + idx * P, 1);
    loss_out[idx] = (mode == kAccum) ? loss_out[idx] + L : L;
  }
}

__global__ __launch_bounds__(256) void apply_kernel(float* __restrict__ theta, const float* __restrict__ grad,
                                                     float lr, int64_t count) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < count) theta[idx] = theta[idx] - lr * grad[idx];
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ dst, float value, int64_t count) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < count) dst[idx] = value;
}

}  // namespace

hipError_t launch_reduce(const float* part, const float* loss_part, int n_heads, int P, int per_head,
                         ReduceMode mode, float* dst, float lr, float* loss_out, hipStream_t stream) {
  const int64_t total = (int64_t)n_heads * per_head;
  const int64_t threads = total > n_heads ? total : n_heads;
  const dim3 grid((unsigned)((threads + 255) / 256));
#define VGGT3_REDUCE_CASE(PP)                                                                         \
  case PP:                                                                                             \
    hipLaunchKernelGGL(reduce_kernel<PP>, grid, dim3(256), 0, stream, part, loss_part, n_heads, per_head, \
                       (int)mode, dst, lr, loss_out);                                                  \
    break;
  switch (P) {
    VGGT3_REDUCE_CASE(1)
    VGGT3_REDUCE_CASE(2)
    VGGT3_REDUCE_CASE(4)
    VGGT3_REDUCE_CASE(8)
    VGGT3_REDUCE_CASE(16)
    VGGT3_REDUCE_CASE(32)
    VGGT3_REDUCE_CASE(64)
    default:
      return hipErrorInvalidValue;
  }
#undef VGGT3_REDUCE_CASE
  return hipGetLastError();
}

hipError_t launch_apply(float* theta, const float* grad, float lr, int64_t count, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(apply_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, theta, grad, lr,
                     count);
  return hipGetLastError();
}

hipError_t launch_fill(float* dst, float value, int64_t count, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, dst, value, count);
  return hipGetLastError();
}

int ttt_num_chunks(int64_t n_tokens, int n_heads, int tile_tokens) {
  const int64_t n_tiles = (n_tokens + tile_tokens - 1) / tile_tokens;
  int64_t target = 512 / (n_heads > 0 ? n_heads : 1);
  if (target < 1) target = 1;
  if (target > n_tiles) target = n_tiles;
  if (target > kMaxChunks) target = kMaxChunks;
  int P = 1;
  while ((int64_t)P * 2 <= target) P *= 2;
  return P;
}

}  // namespace vggt3

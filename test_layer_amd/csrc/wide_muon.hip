// Muon update of the full-width MLP's weights (paper-graph summary "VGG-T3:
// Offline Feed-Forward 3D Reconstruction at Scale", section 3.4 "Muon
// optimizer for inner loop": 5 Newton-Schulz iterations, lr 0.1), for the
// 1024 x 4096 matrices W_g, W_u and the 4096 x 1024 matrix W_d.
//
// NS is the quintic Newton-Schulz map of the Muon optimiser with its published
// coefficients (a, b, c) = (3.4445, -4.7750, 2.0315): X = G / (||G||_F + 1e-7),
// then per step, for a matrix with no more rows than columns,
//   A = X X^T,  B = b A + c A A,  X = a X + B X,
// and for a taller matrix (W_d) the same map on X^T, written without the
// transposes as A = X^T X, X = a X + X B. All in fp32, as the per-head Muon.
//
// The products are fp32 GEMMs on the matrix cores (v_mfma_f32_32x32x2_f32,
// twice the vector FMA rate): 64 x 64 output tiles, 4 waves with a 32 x 32
// sub-tile each, k slices of 16 staged through LDS. Each output takes its k
// terms in ascending order, as a sequential fused multiply-add loop would. A
// GEMM's epilogue is out = alpha * acc + beta * E (E elementwise, same shape as
// out).
#include "bf16_ops.hpp"
#include "kernels.hpp"
#include "wide.hpp"

namespace vggt3 {
namespace wide {
namespace {

constexpr float NS_A = 3.4445f, NS_B = -4.7750f, NS_C = 2.0315f;
constexpr float NS_EPS = 1e-7f;
constexpr int GT = 64, GK = 16;

// C[M x N] = alpha * sum_k A(i, k) B(k, j) + beta * E[i][j], with
// A(i, k) = TA ? A[k * lda + i] : A[i * lda + k] and
// B(k, j) = TB ? B[j * ldb + k] : B[k * ldb + j]; M, N multiples of 64, K of 16.
template <bool TA, bool TB>
__global__ __launch_bounds__(256) void ns_gemm_kernel(const float* __restrict__ A, int64_t lda,
                                                      const float* __restrict__ B, int64_t ldb, int M, int N, int K,
                                                      float alpha, float beta, const float* __restrict__ E,
                                                      float* __restrict__ C) {
  __shared__ float As[GK][GT + 4];
  __shared__ float Bs[GK][GT + 4];
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;  // this wave's 32 x 32 sub-tile
  const int tiles_n = N / GT;
  const int i0 = (blockIdx.x / tiles_n) * GT, j0 = (blockIdx.x % tiles_n) * GT;
  f32x16 acc = {};
  for (int k0 = 0; k0 < K; k0 += GK) {
    if (TA) {  // A(i, k) = A[k * lda + i]: 16 k rows of 64 i
      const int k = t >> 4, i = (t & 15) * 4;
      const f32x4 v = *(const f32x4*)(A + (int64_t)(k0 + k) * lda + i0 + i);
      *(f32x4*)&As[k][i] = v;
    } else {  // A[i * lda + k]: 64 i rows of 16 k
      const int i = t >> 2, k = (t & 3) * 4;
      const f32x4 v = *(const f32x4*)(A + (int64_t)(i0 + i) * lda + k0 + k);
#pragma unroll
      for (int q = 0; q < 4; ++q) As[k + q][i] = v[q];
    }
    if (TB) {  // B[j * ldb + k]: 64 j rows of 16 k
      const int j = t >> 2, k = (t & 3) * 4;
      const f32x4 v = *(const f32x4*)(B + (int64_t)(j0 + j) * ldb + k0 + k);
#pragma unroll
      for (int q = 0; q < 4; ++q) Bs[k + q][j] = v[q];
    } else {  // B[k * ldb + j]: 16 k rows of 64 j
      const int k = t >> 4, j = (t & 15) * 4;
      const f32x4 v = *(const f32x4*)(B + (int64_t)(k0 + k) * ldb + j0 + j);
      *(f32x4*)&Bs[k][j] = v;
    }
    __syncthreads();
    // fp32 MFMA 32x32x2: lane l supplies A(32 wm + l % 32, k + l / 32) and
    // B(k + l / 32, 32 wn + l % 32)
#pragma unroll
    for (int k = 0; k < GK; k += 2) {
      const float a = As[k + (lane >> 5)][32 * wm + (lane & 31)];
      const float b = Bs[k + (lane >> 5)][32 * wn + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // C layout: lane l, register r holds row 8 (r / 4) + 4 (l / 32) + r % 4,
  // column l % 32 of the wave's 32 x 32 sub-tile.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = i0 + 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    const int j = j0 + 32 * wn + (lane & 31);
    const int64_t o = (int64_t)i * N + j;
    float v = alpha * acc[r];
    if (E != nullptr) v = fmaf(beta, E[o], v);
    C[o] = v;
  }
}

// Sum of squares of n values: per-block partials over fixed index ranges.
__global__ __launch_bounds__(256) void sumsq_kernel(const float* __restrict__ x, int64_t n,
                                                    float* __restrict__ partial) {
  __shared__ float red[4];
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = blockIdx.x * per, b1 = b0 + per < n ? b0 + per : n;
  float s = 0.0f;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += 256) s = fmaf(x[i], x[i], s);
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// X = G / (sqrt(sum of the partials) + eps); the partials are summed in a
// fixed order by every block.
__global__ __launch_bounds__(256) void normalize_kernel(const float* __restrict__ g, int64_t n,
                                                        const float* __restrict__ partial, int np,
                                                        float* __restrict__ x) {
  __shared__ float inv;
  if (threadIdx.x == 0) {
    float s = 0.0f;
    for (int i = 0; i < np; ++i) s += partial[i];
    inv = 1.0f / (sqrtf(s) + NS_EPS);
  }
  __syncthreads();
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = g[i] * inv;
}

// theta -= lr * x
__global__ __launch_bounds__(256) void axpy_kernel(float* __restrict__ th, const float* __restrict__ x, float lr,
                                                   int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) th[i] -= lr * x[i];
}

template <bool TA, bool TB>
hipError_t gemm(const float* A, int64_t lda, const float* B, int64_t ldb, int M, int N, int K, float alpha,
                float beta, const float* E, float* C, hipStream_t s) {
  hipLaunchKernelGGL((ns_gemm_kernel<TA, TB>), dim3((M / GT) * (N / GT)), dim3(256), 0, s, A, lda, B, ldb, M, N, K,
                     alpha, beta, E, C);
  return hipGetLastError();
}

constexpr int kNormBlocks = 256;

// One matrix: theta block th (R x Cc, row-major) -= lr * NS(grad block g).
hipError_t ns_one(float* th, const float* g, int R, int Cc, float lr, int ns_steps, float* ws, hipStream_t s) {
  const int64_t n = (int64_t)R * Cc;
  const int small = R < Cc ? R : Cc;
  float* x0 = ws;
  float* x1 = x0 + n;
  float* am = x1 + n;
  float* bm = am + (int64_t)small * small;
  float* partial = bm + (int64_t)small * small;
  hipLaunchKernelGGL(sumsq_kernel, dim3(kNormBlocks), dim3(256), 0, s, g, n, partial);
  hipLaunchKernelGGL(normalize_kernel, dim3(1024), dim3(256), 0, s, g, n, partial, kNormBlocks, x0);
  hipError_t e = hipGetLastError();
  float* x = x0;
  float* xn = x1;
  for (int st = 0; st < ns_steps && e == hipSuccess; ++st) {
    if (R <= Cc) {
      // A = X X^T; B = b A + c A A; X' = B X + a X
      e = gemm<false, true>(x, Cc, x, Cc, R, R, Cc, 1.0f, 0.0f, nullptr, am, s);
      if (e == hipSuccess) e = gemm<false, false>(am, R, am, R, R, R, R, NS_C, NS_B, am, bm, s);
      if (e == hipSuccess) e = gemm<false, false>(bm, R, x, Cc, R, Cc, R, 1.0f, NS_A, x, xn, s);
    } else {
      // A = X^T X; B = b A + c A A; X' = X B + a X
      e = gemm<true, false>(x, Cc, x, Cc, Cc, Cc, R, 1.0f, 0.0f, nullptr, am, s);
      if (e == hipSuccess) e = gemm<false, false>(am, Cc, am, Cc, Cc, Cc, Cc, NS_C, NS_B, am, bm, s);
      if (e == hipSuccess) e = gemm<false, false>(x, Cc, bm, Cc, R, Cc, Cc, 1.0f, NS_A, x, xn, s);
    }
    float* tmp = x;
    x = xn;
    xn = tmp;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(axpy_kernel, dim3(1024), dim3(256), 0, s, th, x, lr, n);
  return hipGetLastError();
}

}  // namespace

size_t muon_workspace_floats(int d, int m) {
  const int64_t n = (int64_t)d * m;
  const int64_t small = d < m ? d : m;
  return (size_t)(2 * n + 2 * small * small + kNormBlocks);
}

hipError_t launch_muon(float* theta, const float* grad, float lr, int d, int m, int ns_steps, float* ws,
                       hipStream_t s) {
  const int64_t dm = (int64_t)d * m;
  hipError_t e = ns_one(theta, grad, d, m, lr, ns_steps, ws, s);                     // W_g [d][m]
  if (e == hipSuccess) e = ns_one(theta + dm, grad + dm, d, m, lr, ns_steps, ws, s);  // W_u [d][m]
  if (e == hipSuccess) e = ns_one(theta + 2 * dm, grad + 2 * dm, m, d, lr, ns_steps, ws, s);  // W_d [m][d]
  return e;
}

}  // namespace wide
}  // namespace vggt3

// Muon update of the fast weights: theta -= lr * NS(g) for every per-head
// weight matrix (paper-graph summary "VGG-T3: Offline Feed-Forward 3D
// Reconstruction at Scale", section 3.4 "Muon optimizer for inner loop": Muon
// with 5 Newton-Schulz iterations, lr 0.1).
//
// NS is the quintic Newton-Schulz orthogonalisation of the Muon optimiser
// (Jordan et al., 2024, the method the pages name), with its published
// coefficients: X = G / (||G||_F + eps), then `steps` times
//   A = X X^T,  B = b A + c A A,  X = a X + B X,
// with X oriented so that it has no more rows than columns. Per head the three
// matrices are W_g [d][m], W_u [d][m] and W_d [m][d]; the last is transposed
// on the way in and out, so every workgroup works on a d x m matrix.
//
// One workgroup per (head, matrix), fp32 throughout, everything in LDS. Each
// of 1024 threads computes 2x2 output blocks of the three matrix products,
// reading its operands four k at a time with 16-byte LDS reads. A matrix's
// update runs on one CU and is bound by its fp32 FMA rate (5 steps of about
// 3 MFLOP each for a 64 x 128 matrix).
#include "bf16_ops.hpp"
#include "kernels.hpp"

namespace vggt3 {
namespace {

constexpr float NS_A = 3.4445f, NS_B = -4.7750f, NS_C = 2.0315f;
constexpr float NS_EPS = 1e-7f;

constexpr int NT = 1024;          // threads per workgroup (four waves per SIMD)
constexpr int BR = 2, BC = 2;      // output block per thread

// out[i][j] = sum_k P(i, k) Q(k, j) for an RA x CB output, in BR x BC blocks
// per thread, with P(i, k) = P[i * ps + k] and Q(k, j) = Q[k * qs + j] (qt =
// false) or Q[j * qs + k] (qt = true). Operands are read four k at a time
// (16-byte LDS reads); each output still sums its k terms in ascending order.
template <int RA, int CB, int KK, bool QT, typename Epi>
__device__ __forceinline__ void matmul_blocks(const float* P, int ps, const float* Q, int qs, Epi epi) {
  static_assert(RA % BR == 0 && CB % BC == 0 && KK % 4 == 0, "blocks");
  constexpr int NB = (RA / BR) * (CB / BC);
  for (int blk = threadIdx.x; blk < NB; blk += NT) {
    const int i0 = (blk / (CB / BC)) * BR, j0 = (blk % (CB / BC)) * BC;
    float acc[BR][BC] = {};
    for (int k = 0; k < KK; k += 4) {
      f32x4 p[BR];
#pragma unroll
      for (int a = 0; a < BR; ++a) p[a] = *reinterpret_cast<const f32x4*>(&P[(i0 + a) * ps + k]);
      if constexpr (QT) {
        f32x4 q[BC];
#pragma unroll
        for (int b = 0; b < BC; ++b) q[b] = *reinterpret_cast<const f32x4*>(&Q[(j0 + b) * qs + k]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int a = 0; a < BR; ++a)
#pragma unroll
            for (int b = 0; b < BC; ++b) acc[a][b] = fmaf(p[a][kk], q[b][kk], acc[a][b]);
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          float q[BC];
#pragma unroll
          for (int b = 0; b < BC; ++b) q[b] = Q[(k + kk) * qs + j0 + b];
#pragma unroll
          for (int a = 0; a < BR; ++a)
#pragma unroll
            for (int b = 0; b < BC; ++b) acc[a][b] = fmaf(p[a][kk], q[b], acc[a][b]);
        }
      }
    }
#pragma unroll
    for (int a = 0; a < BR; ++a)
#pragma unroll
      for (int b = 0; b < BC; ++b) epi(i0 + a, j0 + b, acc[a][b]);
  }
}

template <int R, int CC>
__global__ __launch_bounds__(NT) void muon_apply_kernel(float* __restrict__ theta, const float* __restrict__ grad,
                                                        float lr, int ns_steps) {
  static_assert(R <= CC, "rows <= columns");
  constexpr int XP = CC + 4;  // LDS pitches (16-byte aligned rows)
  constexpr int AP = R + 4;
  constexpr int DM = R * CC;
  constexpr int NWV = NT / 64;
  __shared__ __attribute__((aligned(16))) float X[2][R * XP];
  __shared__ __attribute__((aligned(16))) float A[R * AP];
  __shared__ __attribute__((aligned(16))) float B[R * AP];
  __shared__ float red[NWV];

  const int head = blockIdx.x / 3, mat = blockIdx.x % 3;
  const int tid = threadIdx.x;
  const float* g = grad + ((int64_t)head * 3 + mat) * DM;
  float* th = theta + ((int64_t)head * 3 + mat) * DM;

  float ss = 0.0f;
  for (int idx = tid; idx < DM; idx += NT) {
    const int i = idx / CC, j = idx % CC;
    const float v = mat < 2 ? g[idx] : g[j * R + i];
    X[0][i * XP + j] = v;
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
  for (int i = 0; i < NWV; ++i) tot += red[i];
  const float inv = 1.0f / (sqrtf(tot) + NS_EPS);
  for (int idx = tid; idx < DM; idx += NT) {
    const int i = idx / CC, j = idx % CC;
    X[0][i * XP + j] *= inv;
  }
  __syncthreads();

  int cur = 0;
  for (int s = 0; s < ns_steps; ++s) {
    const float* Xc = X[cur];
    float* Xn = X[cur ^ 1];
    matmul_blocks<R, R, CC, true>(Xc, XP, Xc, XP, [&](int i, int j, float v) { A[i * AP + j] = v; });
    __syncthreads();
    matmul_blocks<R, R, R, false>(A, AP, A, AP,
                                  [&](int i, int j, float v) { B[i * AP + j] = fmaf(NS_C, v, NS_B * A[i * AP + j]); });
    __syncthreads();
    matmul_blocks<R, CC, R, false>(B, AP, Xc, XP,
                                   [&](int i, int j, float v) { Xn[i * XP + j] = fmaf(NS_A, Xc[i * XP + j], v); });
    __syncthreads();
    cur ^= 1;
  }

  const float* Xf = X[cur];
  for (int idx = tid; idx < DM; idx += NT) {
    const int i = idx / CC, j = idx % CC;
    const float o = Xf[i * XP + j];
    if (mat < 2)
      th[idx] -= lr * o;
    else
      th[j * R + i] -= lr * o;
  }
}

}  // namespace

hipError_t launch_muon_apply(float* theta, const float* grad, float lr, int n_heads, int d, int m, int ns_steps,
                             hipStream_t stream) {
  const unsigned n_blocks = (unsigned)(3 * n_heads);
  if (d == 64 && m == 128)
    hipLaunchKernelGGL((muon_apply_kernel<64, 128>), dim3(n_blocks), dim3(NT), 0, stream, theta, grad, lr, ns_steps);
  else if (d == 16 && m == 32)
    hipLaunchKernelGGL((muon_apply_kernel<16, 32>), dim3(n_blocks), dim3(NT), 0, stream, theta, grad, lr, ns_steps);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vggt3

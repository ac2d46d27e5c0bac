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
// One workgroup of 1024 threads per (head, matrix), fp32 throughout,
// everything in LDS; a matrix's update runs on one CU (5 steps of about 2.6
// MFLOP for a 64 x 128 matrix). The (64, 128) matrices use fp32 MFMA, twice
// the vector FMA rate; the small (16, 32) ones use vector FMAs, each thread
// computing 2x2 output blocks with operands read four k at a time.
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

// The (64, 128) matrices on fp32 MFMA (v_mfma_f32_16x16x4_f32, twice the
// vector FMA rate): 16 waves, each owning 16 x 16 output tiles.
//   A operand: lane l holds A[l % 16][k = l / 16]
//   B operand: lane l holds B[k = l / 16][l % 16]
//   C/D:       lane l, register r holds C[4 (l / 16) + r][l % 16]
// The contraction index of MFMA step s and lane quarter q is k = (K/4) q + s,
// so that a lane's operands along a row are consecutive over four steps (one
// 16-byte LDS read); the order in which the products are summed differs from
// the vector kernel's.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc += P(16 ti + i, k) Q(k, 16 tj + j) over k < KK, P rows read four k at
// a time; Q(k, j) = Q[k * qs + j] (column reads) or, with QROW, Q[j * qs + k].
template <int KK, bool QROW>
__device__ __forceinline__ f32x4 mfma_tile(const float* P, int ps, const float* Q, int qs, int ti, int tj, int i,
                                           int q) {
  constexpr int KQ = KK / 4;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const float* prow = P + (16 * ti + i) * ps + KQ * q;
#pragma unroll 2
  for (int s = 0; s < KQ; s += 4) {
    const f32x4 pa = *reinterpret_cast<const f32x4*>(prow + s);
    f32x4 qb;
    if constexpr (QROW) {
      qb = *reinterpret_cast<const f32x4*>(Q + (16 * tj + i) * qs + KQ * q + s);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) qb[u] = Q[(KQ * q + s + u) * qs + 16 * tj + i];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = mfma_f32(pa[u], qb[u], acc);
  }
  return acc;
}

__global__ __launch_bounds__(NT) void muon_apply_mfma_kernel(float* __restrict__ theta,
                                                             const float* __restrict__ grad, float lr,
                                                             int ns_steps) {
  constexpr int R = 64, CC = 128;
  constexpr int XP = CC + 4, AP = R + 4, DM = R * CC;
  constexpr int NWV = NT / 64;
  static_assert(NWV == 16, "one 16 x 16 tile of A per wave");
  __shared__ __attribute__((aligned(16))) float X[2][R * XP];
  __shared__ __attribute__((aligned(16))) float A[R * AP];
  __shared__ __attribute__((aligned(16))) float B[R * AP];
  __shared__ float red[NWV];

  const int head = blockIdx.x / 3, mat = blockIdx.x % 3;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, q = lane >> 4;
  const float* g = grad + ((int64_t)head * 3 + mat) * DM;
  float* th = theta + ((int64_t)head * 3 + mat) * DM;

  float ss = 0.0f;
  for (int idx = tid; idx < DM; idx += NT) {
    const int r = idx / CC, c = idx % CC;
    const float v = mat < 2 ? g[idx] : g[c * R + r];
    X[0][r * XP + c] = v;
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  float tot = 0.0f;
  for (int k = 0; k < NWV; ++k) tot += red[k];
  const float inv = 1.0f / (sqrtf(tot) + NS_EPS);
  for (int idx = tid; idx < DM; idx += NT) {
    const int r = idx / CC, c = idx % CC;
    X[0][r * XP + c] *= inv;
  }
  __syncthreads();

  const int ti = w >> 2, tj = w & 3;  // this wave's 16 x 16 tile of A and B
  int cur = 0;
  for (int s = 0; s < ns_steps; ++s) {
    const float* Xc = X[cur];
    float* Xn = X[cur ^ 1];
    {  // A = X X^T
      const f32x4 acc = mfma_tile<CC, true>(Xc, XP, Xc, XP, ti, tj, i, q);
#pragma unroll
      for (int r = 0; r < 4; ++r) A[(16 * ti + 4 * q + r) * AP + 16 * tj + i] = acc[r];
    }
    __syncthreads();
    {  // B = b A + c A A
      const f32x4 acc = mfma_tile<R, false>(A, AP, A, AP, ti, tj, i, q);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = (16 * ti + 4 * q + r) * AP + 16 * tj + i;
        B[o] = fmaf(NS_C, acc[r], NS_B * A[o]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // X = a X + B X, tiles w and w + 16 of 4 x 8
      const int t = w + 16 * h, xi = t >> 3, xj = t & 7;
      const f32x4 acc = mfma_tile<R, false>(B, AP, Xc, XP, xi, xj, i, q);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = (16 * xi + 4 * q + r) * XP + 16 * xj + i;
        Xn[o] = fmaf(NS_A, Xc[o], acc[r]);
      }
    }
    __syncthreads();
    cur ^= 1;
  }

  const float* Xf = X[cur];
  for (int idx = tid; idx < DM; idx += NT) {
    const int r = idx / CC, c = idx % CC;
    const float o = Xf[r * XP + c];
    if (mat < 2)
      th[idx] -= lr * o;
    else
      th[c * R + r] -= lr * o;
  }
}

}  // namespace

hipError_t launch_muon_apply(float* theta, const float* grad, float lr, int n_heads, int d, int m, int ns_steps,
                             hipStream_t stream) {
  const unsigned n_blocks = (unsigned)(3 * n_heads);
  if (d == 64 && m == 128)
    hipLaunchKernelGGL(muon_apply_mfma_kernel, dim3(n_blocks), dim3(NT), 0, stream, theta, grad, lr, ns_steps);
  else if (d == 16 && m == 32)
    hipLaunchKernelGGL((muon_apply_kernel<16, 32>), dim3(n_blocks), dim3(NT), 0, stream, theta, grad, lr, ns_steps);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vggt3

// fp32 kernels of the TTT write (gradient partials) and read passes.
//
// Same mathematics as the bf16 MFMA path (fast-weight SwiGLU T(x) =
// (silu(x W_g) * (x W_u)) W_d, loss sum_i (1/d)||T(k_i) - v'_i||^2 or, with
// DOT, -sum_i T(k_i) . v'_i ("The dot product loss"), gradient summed per
// token chunk as in Eq. 5 of the paper-graph summary "VGG-T3: Offline
// Feed-Forward 3D Reconstruction at Scale", section 3.4), evaluated
// entirely in fp32 on the vector ALUs. This path serves the fp32 mode (tight
// tolerances, small heads); it stages the head's weights and every per-tile
// intermediate in LDS and lets each thread own a fixed set of outputs.
#include "common.hpp"
#include "kernels.hpp"

namespace vggt3 {
namespace {

template <int D, int M>
struct F32Cfg {
  static constexpr int TT = 16;  // tokens per tile
  static constexpr int DM = D * M;
  static constexpr int PER_HEAD = 3 * DM;
  static constexpr int NACC = PER_HEAD / 256;
};

__device__ __forceinline__ float sigmoid_f32(float x) { return 1.0f / (1.0f + __expf(-x)); }

template <int D, int M, bool DOT>
__global__ __launch_bounds__(256, 1) void grad_partial_f32_kernel(const float* __restrict__ K,
                                                                const float* __restrict__ Vp,
                                                                const float* __restrict__ theta,
                                                                float* __restrict__ part,
                                                                float* __restrict__ loss_part,
                                                                int64_t n_tokens, int n_heads, int P,
                                                                int64_t n_blocks) {
  using Cfg = F32Cfg<D, M>;
  constexpr int TT = Cfg::TT, DM = Cfg::DM, PER_HEAD = Cfg::PER_HEAD, NACC = Cfg::NACC;
  __shared__ float W[PER_HEAD];
  __shared__ float Ks[TT * D], Vs[TT * D], dYs[TT * D];
  __shared__ float Hs[TT * M], As[TT * M], GPs[TT * M], dGs[TT * M], dUs[TT * M];
  __shared__ float red[4];

  const int64_t blk = xcd_remap(blockIdx.x, n_blocks);
  const int head = (int)(blk / P);
  const int chunk = (int)(blk % P);
  const int tid = threadIdx.x;
  const int64_t C = (int64_t)n_heads * D;
  const float* th = theta + (int64_t)head * PER_HEAD;
  for (int i = tid; i < PER_HEAD; i += 256) W[i] = th[i];
  const float* Wg = W;
  const float* Wu = W + DM;
  const float* Wd = W + 2 * DM;

  float acc[NACC];
#pragma unroll
  for (int q = 0; q < NACC; ++q) acc[q] = 0.0f;
  float loss = 0.0f;

  const int64_t n_tiles = (n_tokens + TT - 1) / TT;
  const int64_t tile_begin = n_tiles * chunk / P;
  const int64_t tile_end = n_tiles * (chunk + 1) / P;
  __syncthreads();

  for (int64_t tile = tile_begin; tile < tile_end; ++tile) {
    const int64_t tok0 = tile * TT;
    for (int i = tid; i < TT * D; i += 256) {
      const int t = i / D, c = i % D;
      const int64_t tok = tok0 + t;
      const bool ok = tok < n_tokens;
      Ks[i] = ok ? K[tok * C + (int64_t)head * D + c] : 0.0f;
      Vs[i] = ok ? Vp[tok * C + (int64_t)head * D + c] : 0.0f;
    }
    __syncthreads();
    for (int i = tid; i < TT * M; i += 256) {
      const int t = i / M, j = i % M;
      float g = 0.0f, u = 0.0f;
      for (int e = 0; e < D; ++e) {
        g = fmaf(Ks[t * D + e], Wg[e * M + j], g);
        u = fmaf(Ks[t * D + e], Wu[e * M + j], u);
      }
      const float s = sigmoid_f32(g);
      const float a = g * s;
      const float h = a * u;
      Hs[i] = h;
      As[i] = a;
      GPs[i] = u * s + h * (1.0f - s);
    }
    __syncthreads();
    for (int i = tid; i < TT * D; i += 256) {
      const int t = i / D, o = i % D;
      float y = 0.0f;
      for (int j = 0; j < M; ++j) y = fmaf(Hs[t * M + j], Wd[j * D + o], y);
      if (DOT) {  // L = -sum y . v', dL/dy = -v'
        loss = fmaf(-y, Vs[i], loss);
        dYs[i] = -Vs[i];
      } else {
        const float R = y - Vs[i];
        loss = fmaf(R, R, loss);
        dYs[i] = (2.0f / D) * R;
      }
    }
    __syncthreads();
    for (int i = tid; i < TT * M; i += 256) {
      const int t = i / M, j = i % M;
      float dh = 0.0f;
      for (int o = 0; o < D; ++o) dh = fmaf(dYs[t * D + o], Wd[j * D + o], dh);
      dUs[i] = dh * As[i];
      dGs[i] = dh * GPs[i];
    }
    __syncthreads();
    // Thread tid owns parameters tid + 256q; DM is a multiple of 256, so each
    // q falls wholly in one of the three matrices.
    static_assert(DM % 256 == 0, "parameter blocks must be whole multiples of the workgroup");
    for (int t = 0; t < TT; ++t) {
#pragma unroll
      for (int q = 0; q < NACC; ++q) {
        const int idx = tid + 256 * q;
        if (q < DM / 256) {
          const int e = idx / M, j = idx % M;
          acc[q] = fmaf(Ks[t * D + e], dGs[t * M + j], acc[q]);
        } else if (q < 2 * DM / 256) {
          const int e = (idx - DM) / M, j = (idx - DM) % M;
          acc[q] = fmaf(Ks[t * D + e], dUs[t * M + j], acc[q]);
        } else {
          const int j = (idx - 2 * DM) / D, o = (idx - 2 * DM) % D;
          acc[q] = fmaf(Hs[t * M + j], dYs[t * D + o], acc[q]);
        }
      }
    }
    __syncthreads();
  }

  float* out = part + ((int64_t)head * P + chunk) * PER_HEAD;
#pragma unroll
  for (int q = 0; q < NACC; ++q) out[tid + 256 * q] = acc[q];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) loss += __shfl_xor(loss, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = loss;
  __syncthreads();
  if (tid == 0)
    loss_part[(int64_t)head * P + chunk] = ((red[0] + red[1]) + (red[2] + red[3])) * (DOT ? 1.0f : 1.0f / D);
}

template <int D, int M>
__global__ __launch_bounds__(256) void read_f32_kernel(const float* __restrict__ Q,
                                                        const float* __restrict__ theta,
                                                        float* __restrict__ O, int64_t n_tokens,
                                                        int n_heads, int P, int64_t n_blocks) {
  using Cfg = F32Cfg<D, M>;
  constexpr int TT = 32, DM = Cfg::DM, PER_HEAD = Cfg::PER_HEAD;
  __shared__ float W[PER_HEAD];
  __shared__ float Qs[TT * D], Hs[TT * M];
  const int64_t blk = xcd_remap(blockIdx.x, n_blocks);
  const int head = (int)(blk / P);
  const int chunk = (int)(blk % P);
  const int tid = threadIdx.x;
  const int64_t C = (int64_t)n_heads * D;
  const float* th = theta + (int64_t)head * PER_HEAD;
  for (int i = tid; i < PER_HEAD; i += 256) W[i] = th[i];
  const float* Wg = W;
  const float* Wu = W + DM;
  const float* Wd = W + 2 * DM;
  const int64_t n_tiles = (n_tokens + TT - 1) / TT;
  const int64_t tile_begin = n_tiles * chunk / P;
  const int64_t tile_end = n_tiles * (chunk + 1) / P;
  __syncthreads();
  for (int64_t tile = tile_begin; tile < tile_end; ++tile) {
    const int64_t tok0 = tile * TT;
    for (int i = tid; i < TT * D; i += 256) {
      const int64_t tok = tok0 + i / D;
      Qs[i] = tok < n_tokens ? Q[tok * C + (int64_t)head * D + i % D] : 0.0f;
    }
    __syncthreads();
    for (int i = tid; i < TT * M; i += 256) {
      const int t = i / M, j = i % M;
      float g = 0.0f, u = 0.0f;
      for (int e = 0; e < D; ++e) {
        g = fmaf(Qs[t * D + e], Wg[e * M + j], g);
        u = fmaf(Qs[t * D + e], Wu[e * M + j], u);
      }
      Hs[i] = g * sigmoid_f32(g) * u;
    }
    __syncthreads();
    for (int i = tid; i < TT * D; i += 256) {
      const int t = i / D, o = i % D;
      const int64_t tok = tok0 + t;
      float y = 0.0f;
      for (int j = 0; j < M; ++j) y = fmaf(Hs[t * M + j], Wd[j * D + o], y);
      if (tok < n_tokens) O[tok * C + (int64_t)head * D + o] = y;
    }
    __syncthreads();
  }
}

template <int D, int M>
hipError_t launch_grad_f32_t(const float* K, const float* Vp, const float* theta, float* part,
                             float* loss_part, int64_t n_tokens, int n_heads, int P, bool dot,
                             hipStream_t stream) {
  const int64_t n_blocks = (int64_t)n_heads * P;
  if (dot)
    hipLaunchKernelGGL((grad_partial_f32_kernel<D, M, true>), dim3((unsigned)n_blocks), dim3(256), 0, stream, K,
                       Vp, theta, part, loss_part, n_tokens, n_heads, P, n_blocks);
  else
    hipLaunchKernelGGL((grad_partial_f32_kernel<D, M, false>), dim3((unsigned)n_blocks), dim3(256), 0, stream, K,
                       Vp, theta, part, loss_part, n_tokens, n_heads, P, n_blocks);
  return hipGetLastError();
}

template <int D, int M>
hipError_t launch_read_f32_t(const float* Q, const float* theta, float* O, int64_t n_tokens, int n_heads,
                             hipStream_t stream) {
  const int64_t n_tiles = (n_tokens + 31) / 32;
  int64_t P = (512 + n_heads - 1) / n_heads;
  if (P > n_tiles) P = n_tiles;
  if (P < 1) P = 1;
  const int64_t n_blocks = (int64_t)n_heads * P;
  hipLaunchKernelGGL((read_f32_kernel<D, M>), dim3((unsigned)n_blocks), dim3(256), 0, stream, Q, theta, O,
                     n_tokens, n_heads, (int)P, n_blocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grad_partial_f32(const void* K, const void* Vp, const float* theta, float* part,
                                   float* loss_part, int64_t n_tokens, int n_heads, int d, int m, int P,
                                   bool dot, hipStream_t stream) {
  const float* k = static_cast<const float*>(K);
  const float* v = static_cast<const float*>(Vp);
  if (d == 16 && m == 32)
    return launch_grad_f32_t<16, 32>(k, v, theta, part, loss_part, n_tokens, n_heads, P, dot, stream);
  if (d == 64 && m == 128)
    return launch_grad_f32_t<64, 128>(k, v, theta, part, loss_part, n_tokens, n_heads, P, dot, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_read_f32(const void* Q, const float* theta, void* O, int64_t n_tokens, int n_heads, int d,
                           int m, hipStream_t stream) {
  const float* q = static_cast<const float*>(Q);
  float* o = static_cast<float*>(O);
  if (d == 16 && m == 32) return launch_read_f32_t<16, 32>(q, theta, o, n_tokens, n_heads, stream);
  if (d == 64 && m == 128) return launch_read_f32_t<64, 128>(q, theta, o, n_tokens, n_heads, stream);
  return hipErrorInvalidValue;
}

}  // namespace vggt3

// fp32 kernels of the TTT write (gradient partials) and read passes.
//
// Same mathematics as the bf16 MFMA path (fast-weight SwiGLU T(x) =
// (silu(x W_g) * (x W_u)) W_d, loss sum_i (1/d)||T(k_i) - v'_i||^2 or, with
// DOT, -sum_i T(k_i) . v'_i ("The dot product loss"), gradient summed per
// token chunk as in Eq. 5 of the paper-graph summary "VGG-T3: Offline
// Feed-Forward 3D Reconstruction at Scale", section 3.4), evaluated
// entirely in fp32. This path serves the fp32 mode (tight tolerances). The
// (64, 128) heads run on the matrix cores (v_mfma_f32_16x16x4_f32, twice the
// vector FMA rate): that instruction adds its k terms to the accumulator one
// after another as fused multiply-adds, so with every product summed in
// ascending k the results are bitwise those of a plain fused multiply-add loop.
// The small (16, 32) heads use vector kernels that stage the head's weights and
// every per-tile intermediate in LDS and let each thread own a fixed set of
// outputs.
// With BF the token tensors (K, V', Q, O) are bf16: they are widened exactly
// on load and O is rounded to bf16 (ties to even) on store; the arithmetic
// stays fp32. This serves the bf16 mode at the small (16, 32) head shape,
// whose per-head tiles are too narrow for the 32-wide MFMA kernels.
#include "common.hpp"
#include "kernels.hpp"

namespace vggt3 {
namespace {

template <int D, int M>
struct F32Cfg {
  static constexpr int TT = 16;  // tokens per tile
  static_assert(TT == kGradTileF32, "the chunking cuts tokens in units of this tile");
  static constexpr int DM = D * M;
  static constexpr int PER_HEAD = 3 * DM;
  static constexpr int NACC = PER_HEAD / 256;
};

__device__ __forceinline__ float sigmoid_f32(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Token element i of a bf16 (BF) or fp32 tensor, as fp32.
template <bool BF>
__device__ __forceinline__ float ld_tok(const void* p, int64_t i) {
  if constexpr (BF) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

template <int D, int M, bool DOT, bool BF>
__global__ __launch_bounds__(256, 1) void grad_partial_f32_kernel(const void* __restrict__ K,
                                                                const void* __restrict__ Vp,
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
      Ks[i] = ok ? ld_tok<BF>(K, tok * C + (int64_t)head * D + c) : 0.0f;
      Vs[i] = ok ? ld_tok<BF>(Vp, tok * C + (int64_t)head * D + c) : 0.0f;
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

template <int D, int M, bool BF>
__global__ __launch_bounds__(256) void read_f32_kernel(const void* __restrict__ Q,
                                                        const float* __restrict__ theta,
                                                        void* __restrict__ O, int64_t n_tokens,
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
      Qs[i] = tok < n_tokens ? ld_tok<BF>(Q, tok * C + (int64_t)head * D + i % D) : 0.0f;
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
      if (tok < n_tokens) {
        const int64_t at = tok * C + (int64_t)head * D + o;
        if constexpr (BF) static_cast<uint16_t*>(O)[at] = f32_to_bf16_bits(y);
        else static_cast<float*>(O)[at] = y;
      }
    }
    __syncthreads();
  }
}

// fp32 read for (d, m) = (64, 128) on the matrix cores (v_mfma_f32_16x16x4_f32).
// The fp32 MFMA adds its k terms to the accumulator one after another as fused
// multiply-adds, so each output is bitwise the vector loop's sum over ascending
// k. 4 waves; per 32-token tile, wave w computes G and U for hidden units
// 32w .. 32w + 31 of both 16-token halves, the SwiGLU, then two 16 x 16
// tiles of Y.
//   A operand: lane l holds A[l % 16][k = l / 16]
//   B operand: lane l holds B[k = l / 16][l % 16]
//   C/D:       lane l, register r holds C[4 (l / 16) + r][l % 16]
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256) void read_f32_mfma_kernel(const float* __restrict__ Q,
                                                            const float* __restrict__ theta,
                                                            float* __restrict__ O, int64_t n_tokens, int n_heads,
                                                            int P, int64_t n_blocks) {
  constexpr int D = 64, M = 128, TT = 32, DM = D * M, PER_HEAD = 3 * DM;
  constexpr int QP = D + 4, HP = M + 4;
  __shared__ float W[PER_HEAD];
  __shared__ float Qs[TT * QP], Hs[TT * HP];
  const int64_t blk = xcd_remap(blockIdx.x, n_blocks);
  const int head = (int)(blk / P);
  const int chunk = (int)(blk % P);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q = lane >> 4;
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
    for (int i = tid; i < TT * D / 4; i += 256) {
      const int t = i / (D / 4), c4 = 4 * (i % (D / 4));
      const int64_t tok = tok0 + t;
      f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
      if (tok < n_tokens) v = *reinterpret_cast<const f32x4*>(Q + tok * C + (int64_t)head * D + c4);
      *reinterpret_cast<f32x4*>(&Qs[t * QP + c4]) = v;
    }
    __syncthreads();
    // G, U for tokens 16 tb + 4 q + r, hidden units 32 w + 16 jb + l16.
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 g[2] = {f32x4{}, f32x4{}}, u[2] = {f32x4{}, f32x4{}};
      for (int k = 0; k < D; k += 4) {
        const float a = Qs[(16 * tb + l16) * QP + k + q];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const int j = 32 * w + 16 * jb + l16;
          g[jb] = mfma_f32(a, Wg[(k + q) * M + j], g[jb]);
          u[jb] = mfma_f32(a, Wu[(k + q) * M + j], u[jb]);
        }
      }
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Hs[(16 * tb + 4 * q + r) * HP + 32 * w + 16 * jb + l16] = g[jb][r] * sigmoid_f32(g[jb][r]) * u[jb][r];
    }
    __syncthreads();
    // Y tiles (tokens 16 tb.., outputs 16 ob..): tb = w >> 1, ob = 2 (w & 1) + b.
    {
      const int tb = w >> 1;
      f32x4 y[2] = {f32x4{}, f32x4{}};
      for (int k = 0; k < M; k += 4) {
        const float a = Hs[(16 * tb + l16) * HP + k + q];
#pragma unroll
        for (int b = 0; b < 2; ++b) y[b] = mfma_f32(a, Wd[(k + q) * D + 16 * (2 * (w & 1) + b) + l16], y[b]);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t tok = tok0 + 16 * tb + 4 * q + r;
          if (tok < n_tokens) O[tok * C + (int64_t)head * D + 16 * (2 * (w & 1) + b) + l16] = y[b][r];
        }
    }
    __syncthreads();
  }
}

// fp32 gradient partials for (d, m) = (64, 128) on the matrix cores, the
// same arithmetic as grad_partial_f32_kernel: every product sums its k terms
// in ascending order (so the partials are bitwise that kernel's), and the
// elementwise steps are the same expressions. 4 waves; per 16-token tile, wave w
// computes G, U and dH for hidden units 32w .. 32w + 31, Y for outputs 16w ..
// 16w + 15, and owns 24 of the 96 16 x 16 tiles of the weight gradients
// (W_g and W_u rows 16w .. 16w + 15, W_d rows 32w .. 32w + 31).
template <bool DOT>
__global__ __launch_bounds__(256) void grad_partial_f32_mfma_kernel(const float* __restrict__ K,
                                                                    const float* __restrict__ Vp,
                                                                    const float* __restrict__ theta,
                                                                    float* __restrict__ part,
                                                                    float* __restrict__ loss_part, int64_t n_tokens,
                                                                    int n_heads, int P, int64_t n_blocks) {
  constexpr int D = 64, M = 128, TT = 16, DM = D * M, PER_HEAD = 3 * DM;
  constexpr int KP = D + 4, HP = M + 4;
  __shared__ float W[PER_HEAD];
  __shared__ float Ks[TT * KP], Vs[TT * KP], dYs[TT * KP];
  __shared__ float Hs[TT * HP], As[TT * HP], GPs[TT * HP], dGs[TT * HP], dUs[TT * HP];
  __shared__ float red[4];

  const int64_t blk = xcd_remap(blockIdx.x, n_blocks);
  const int head = (int)(blk / P);
  const int chunk = (int)(blk % P);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t C = (int64_t)n_heads * D;
  const float* th = theta + (int64_t)head * PER_HEAD;
  for (int i = tid; i < PER_HEAD; i += 256) W[i] = th[i];
  const float* Wg = W;
  const float* Wu = W + DM;
  const float* Wd = W + 2 * DM;

  f32x4 aG[8], aU[8], aD[8];  // W_g / W_u tiles (16w.., 16jb..), W_d tiles (32w + 16(b/4).., 16(b%4)..)
#pragma unroll
  for (int b = 0; b < 8; ++b) aG[b] = aU[b] = aD[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float loss = 0.0f;

  const int64_t n_tiles = (n_tokens + TT - 1) / TT;
  const int64_t tile_begin = n_tiles * chunk / P;
  const int64_t tile_end = n_tiles * (chunk + 1) / P;
  __syncthreads();

  for (int64_t tile = tile_begin; tile < tile_end; ++tile) {
    const int64_t tok0 = tile * TT;
    {  // stage K and V' (zero rows past the end): 256 threads x 16 bytes per tensor
      const int t = tid >> 4, c4 = 4 * (tid & 15);
      const int64_t tok = tok0 + t;
      f32x4 kv = {0.0f, 0.0f, 0.0f, 0.0f}, vv = {0.0f, 0.0f, 0.0f, 0.0f};
      if (tok < n_tokens) {
        kv = *reinterpret_cast<const f32x4*>(K + tok * C + (int64_t)head * D + c4);
        vv = *reinterpret_cast<const f32x4*>(Vp + tok * C + (int64_t)head * D + c4);
      }
      *reinterpret_cast<f32x4*>(&Ks[t * KP + c4]) = kv;
      *reinterpret_cast<f32x4*>(&Vs[t * KP + c4]) = vv;
    }
    __syncthreads();
    {  // G, U (tokens 4q + r, hidden units 32w + 16jb + l16) and the SwiGLU
      f32x4 g[2] = {f32x4{}, f32x4{}}, u[2] = {f32x4{}, f32x4{}};
      for (int k = 0; k < D; k += 4) {
        const float a = Ks[l16 * KP + k + q];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const int j = 32 * w + 16 * jb + l16;
          g[jb] = mfma_f32(a, Wg[(k + q) * M + j], g[jb]);
          u[jb] = mfma_f32(a, Wu[(k + q) * M + j], u[jb]);
        }
      }
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = (4 * q + r) * HP + 32 * w + 16 * jb + l16;
          const float gg = g[jb][r], uu = u[jb][r];
          const float s = sigmoid_f32(gg);
          const float a = gg * s;
          const float h = a * uu;
          Hs[i] = h;
          As[i] = a;
          GPs[i] = uu * s + h * (1.0f - s);
        }
    }
    __syncthreads();
    {  // Y (tokens 4q + r, outputs 16w + l16), the loss and dL/dY
      f32x4 y = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int k = 0; k < M; k += 4) y = mfma_f32(Hs[l16 * HP + k + q], Wd[(k + q) * D + 16 * w + l16], y);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = (4 * q + r) * KP + 16 * w + l16;
        if (DOT) {
          loss = fmaf(-y[r], Vs[i], loss);
          dYs[i] = -Vs[i];
        } else {
          const float R = y[r] - Vs[i];
          loss = fmaf(R, R, loss);
          dYs[i] = (2.0f / D) * R;
        }
      }
    }
    __syncthreads();
    {  // dH (tokens 4q + r, hidden units 32w + 16jb + l16); dU, dG
      f32x4 dh[2] = {f32x4{}, f32x4{}};
      for (int k = 0; k < D; k += 4) {
        const float a = dYs[l16 * KP + k + q];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) dh[jb] = mfma_f32(a, Wd[(32 * w + 16 * jb + l16) * D + k + q], dh[jb]);
      }
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = (4 * q + r) * HP + 32 * w + 16 * jb + l16;
          dUs[i] = dh[jb][r] * As[i];
          dGs[i] = dh[jb][r] * GPs[i];
        }
    }
    __syncthreads();
    // Weight gradients over the tile's 16 tokens, in token order.
#pragma unroll
    for (int k = 0; k < TT; k += 4) {
      const float ke = Ks[(k + q) * KP + 16 * w + l16];  // K^T row 16w + l16
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) {
        aG[jb] = mfma_f32(ke, dGs[(k + q) * HP + 16 * jb + l16], aG[jb]);
        aU[jb] = mfma_f32(ke, dUs[(k + q) * HP + 16 * jb + l16], aU[jb]);
      }
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const float hj = Hs[(k + q) * HP + 32 * w + 16 * (b >> 2) + l16];  // H^T row
        aD[b] = mfma_f32(hj, dYs[(k + q) * KP + 16 * (b & 3) + l16], aD[b]);
      }
    }
    __syncthreads();
  }

  float* out = part + ((int64_t)head * P + chunk) * PER_HEAD;
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = 16 * w + 4 * q + r;
      out[e * M + 16 * b + l16] = aG[b][r];
      out[DM + e * M + 16 * b + l16] = aU[b][r];
      const int j = 32 * w + 16 * (b >> 2) + 4 * q + r;
      out[2 * DM + j * D + 16 * (b & 3) + l16] = aD[b][r];
    }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) loss += __shfl_xor(loss, off, 64);
  if (lane == 0) red[w] = loss;
  __syncthreads();
  if (tid == 0)
    loss_part[(int64_t)head * P + chunk] = ((red[0] + red[1]) + (red[2] + red[3])) * (DOT ? 1.0f : 1.0f / D);
}

template <int D, int M, bool BF>
hipError_t launch_grad_f32_t(const void* K, const void* Vp, const float* theta, float* part,
                             float* loss_part, int64_t n_tokens, int n_heads, int P, bool dot,
                             hipStream_t stream) {
  const int64_t n_blocks = (int64_t)n_heads * P;
  if (dot)
    hipLaunchKernelGGL((grad_partial_f32_kernel<D, M, true, BF>), dim3((unsigned)n_blocks), dim3(256), 0, stream,
                       K, Vp, theta, part, loss_part, n_tokens, n_heads, P, n_blocks);
  else
    hipLaunchKernelGGL((grad_partial_f32_kernel<D, M, false, BF>), dim3((unsigned)n_blocks), dim3(256), 0, stream,
                       K, Vp, theta, part, loss_part, n_tokens, n_heads, P, n_blocks);
  return hipGetLastError();
}

template <int D, int M, bool BF>
hipError_t launch_read_f32_t(const void* Q, const float* theta, void* O, int64_t n_tokens, int n_heads,
                             hipStream_t stream) {
  const int64_t n_tiles = (n_tokens + 31) / 32;
  int64_t P = (512 + n_heads - 1) / n_heads;
  if (P > n_tiles) P = n_tiles;
  if (P < 1) P = 1;
  const int64_t n_blocks = (int64_t)n_heads * P;
  hipLaunchKernelGGL((read_f32_kernel<D, M, BF>), dim3((unsigned)n_blocks), dim3(256), 0, stream, Q, theta, O,
                     n_tokens, n_heads, (int)P, n_blocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grad_partial_f32(const void* K, const void* Vp, const float* theta, float* part,
                                   float* loss_part, int64_t n_tokens, int n_heads, int d, int m, int P,
                                   bool dot, bool bf16_tokens, hipStream_t stream) {
  if (d == 16 && m == 32)
    return bf16_tokens
               ? launch_grad_f32_t<16, 32, true>(K, Vp, theta, part, loss_part, n_tokens, n_heads, P, dot, stream)
               : launch_grad_f32_t<16, 32, false>(K, Vp, theta, part, loss_part, n_tokens, n_heads, P, dot, stream);
  if (d == 64 && m == 128 && !bf16_tokens) {
    const int64_t n_blocks = (int64_t)n_heads * P;
    const float* Kf = static_cast<const float*>(K);
    const float* Vf = static_cast<const float*>(Vp);
    if (dot)
      hipLaunchKernelGGL(grad_partial_f32_mfma_kernel<true>, dim3((unsigned)n_blocks), dim3(256), 0, stream, Kf, Vf,
                         theta, part, loss_part, n_tokens, n_heads, P, n_blocks);
    else
      hipLaunchKernelGGL(grad_partial_f32_mfma_kernel<false>, dim3((unsigned)n_blocks), dim3(256), 0, stream, Kf, Vf,
                         theta, part, loss_part, n_tokens, n_heads, P, n_blocks);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

hipError_t launch_read_f32(const void* Q, const float* theta, void* O, int64_t n_tokens, int n_heads, int d,
                           int m, bool bf16_tokens, hipStream_t stream) {
  if (d == 16 && m == 32)
    return bf16_tokens ? launch_read_f32_t<16, 32, true>(Q, theta, O, n_tokens, n_heads, stream)
                       : launch_read_f32_t<16, 32, false>(Q, theta, O, n_tokens, n_heads, stream);
  if (d == 64 && m == 128 && !bf16_tokens) {
    const int64_t n_tiles = (n_tokens + 31) / 32;
    int64_t P = (512 + n_heads - 1) / n_heads;
    if (P > n_tiles) P = n_tiles;
    if (P < 1) P = 1;
    const int64_t n_blocks = (int64_t)n_heads * P;
    hipLaunchKernelGGL(read_f32_mfma_kernel, dim3((unsigned)n_blocks), dim3(256), 0, stream,
                       static_cast<const float*>(Q), theta, static_cast<float*>(O), n_tokens, n_heads, (int)P, n_blocks);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace vggt3

// bf16-MFMA kernels of the TTT write (gradient partials) and read passes for
// the VGGT shape: per head d = 64 inputs/outputs, m = 128 hidden units.
//
// Fast-weight MLP per head (paper-graph summary "VGG-T3: Offline Feed-Forward
// 3D Reconstruction at Scale", section 3.4 "TTT MLP Architecture and Inner
// Optimization", bias-free SwiGLU):   T(x) = (silu(x W_g) * (x W_u)) W_d.
// Inner loss (Eq. 3 of the same section with a squared error), per head:
//   L = sum_i (1/d) ||T(k_i) - v'_i||^2.
// Its gradient is a sum of per-token terms (Eq. 5, "Large-Scale Inference
// Strategies"), computed here as one fp32 partial per (head, token chunk).
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, see common.hpp): a C/D tile keeps its
// rows in registers and its columns across lanes. Any contraction can take a C
// tile straight back as an operand as long as it contracts over the tile's rows
// (the order of the contraction index is free, and both operands use the same
// permutation). The write pass keeps tokens in rows (registers), so the three
// weight-gradient contractions (over tokens) take H, dG and dU straight from
// registers; H and dY are transposed once through LDS for the two contractions
// over hidden units and outputs.
#include "common.hpp"
#include "kernels.hpp"

namespace vggt3 {
namespace {

constexpr int D = 64;        // head dim (inputs and outputs of T)
constexpr int M = 128;       // hidden units
constexpr int T = 64;        // tokens per tile of the write pass
constexpr int KP = D + 8;    // LDS row pitch (elements) of 64-wide tiles
constexpr int HP = M + 8;    // LDS row pitch of 128-wide tiles
constexpr int DM = D * M;
constexpr int PER_HEAD = 3 * DM;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 ld_op(const uint16_t* p) { return as_bf16x8(ld16(p)); }

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  u32x4 q;
  q[0] = pack_bf16x2(v[0], v[1]);
  q[1] = pack_bf16x2(v[2], v[3]);
  q[2] = pack_bf16x2(v[4], v[5]);
  q[3] = pack_bf16x2(v[6], v[7]);
  return as_bf16x8(q);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Write pass: fp32 gradient partial of one (head, chunk).
//
// Workgroup = 4 waves; wave w owns hidden units [32w, 32w+32) for G, U, H, dH,
// dG, dU and the matching slices of the three gradients:
//   gW_g[:, hid], gW_u[:, hid] (64 x 32 each) and gW_d[hid, :] (32 x 64).
// Per 64-token tile:
//   1. K, V' tiles -> LDS (row-major [token][channel]).
//   2. G, U = K W_g, K W_u for the wave's 32 hidden units (tokens = MFMA rows).
//   3. VALU: s = sigmoid(G), A = G s, H = A U, gp = U silu'(G) = U s + H (1 - s);
//      H -> LDS (row-major, for the Y contraction over hidden units).
//   4. Wave w computes the Y tile (tokens 32*(w/2).., outputs 32*(w%2)..) =
//      H W_d; R = Y - V', dY = (2/d) R -> LDS; loss += |R|^2.
//   5. dH = dY W_d^T for the wave's hidden units; dU = dH A, dG = dH gp.
//   6. gW_d += H^T dY, gW_g += K^T dG, gW_u += K^T dU (tokens = MFMA k).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 1) void grad_partial_bf16_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Vp, const float* __restrict__ theta,
    float* __restrict__ part, float* __restrict__ loss_part, int64_t n_tokens, int n_heads, int P,
    int64_t n_blocks) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[T * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[T * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Hs[T * HP];
  __shared__ __attribute__((aligned(16))) uint16_t dYs[T * KP];
  __shared__ float red[4];

  const int64_t blk = xcd_remap(blockIdx.x, n_blocks);
  const int head = (int)(blk / P);
  const int chunk = (int)(blk % P);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t C = (int64_t)n_heads * D;

  const float* th = theta + (int64_t)head * PER_HEAD;
  const float* Wg = th;
  const float* Wu = th + DM;
  const float* Wd = th + 2 * DM;

  // Weight operands held in registers for the whole chunk (bf16, RNE from fp32).
  bf16x8 WgB[4], WuB[4], WdB[8], WdTB[4];
  {
    const int hid = 32 * w + l32;
    const int ob = w & 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float g[8], u[8], dt[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = 16 * ks + 8 * hh + j;
        g[j] = Wg[e * M + hid];
        u[j] = Wu[e * M + hid];
        dt[j] = Wd[hid * D + e];  // W_d[hid][o = e]
      }
      WgB[ks] = pack8(g);
      WuB[ks] = pack8(u);
      WdTB[ks] = pack8(dt);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = Wd[(16 * ks + 8 * hh + j) * D + 32 * ob + l32];
      WdB[ks] = pack8(v);
    }
  }

  f32x16 accWd[2], accWg[2], accWu[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    accWd[i] = f32x16{};
    accWg[i] = f32x16{};
    accWu[i] = f32x16{};
  }
  float loss = 0.0f;

  const int64_t n_tiles = (n_tokens + T - 1) / T;
  const int64_t tile_begin = n_tiles * chunk / P;
  const int64_t tile_end = n_tiles * (chunk + 1) / P;

  for (int64_t tile = tile_begin; tile < tile_end; ++tile) {
    const int64_t tok0 = tile * T;
    // 1. stage K and V' (zero rows past the end contribute nothing: G = U = 0
    //    gives H = Y = 0, and V' = 0 gives R = 0).
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const int c = (tid & 7) * 8;
      const int64_t tok = tok0 + r;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (tok < n_tokens) {
        const int64_t off = tok * C + (int64_t)head * D + c;
        kv = ld16(K + off);
        vv = ld16(Vp + off);
      }
      st16(&Ks[r * KP + c], kv);
      st16(&Vs[r * KP + c], vv);
    }
    __syncthreads();

    // 2. G, U for this wave's hidden units; element (mt, r) is token
    //    32mt + 8(r/4) + 4hh + r%4, hidden unit 32w + l32.
    f32x16 accG[2], accU[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      accG[mt] = f32x16{};
      accU[mt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = ld_op(&Ks[(32 * mt + l32) * KP + 16 * ks + 8 * hh]);
        accG[mt] = mfma32(a, WgB[ks], accG[mt]);
        accU[mt] = mfma32(a, WuB[ks], accU[mt]);
      }
    }

    // 3. SwiGLU elementwise.
    float Aa[2][16], GP[2][16], Hf[2][16];
    const int hid = 32 * w + l32;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float g = accG[mt][r];
        const float u = accU[mt][r];
        const float s = sigmoid_fast(g);
        const float a = g * s;
        const float h = a * u;
        Aa[mt][r] = a;
        Hf[mt][r] = h;
        GP[mt][r] = u * s + h * (1.0f - s);
        const int t = 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
        Hs[t * HP + hid] = f32_to_bf16_bits(h);
      }
    }
    bf16x8 Hop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Hop[ks] = pack8(&Hf[ks >> 1][8 * (ks & 1)]);
    __syncthreads();

    // 4. Y tile, residual, dY.
    {
      const int tb = w >> 1, ob = w & 1;
      f32x16 accY = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 a = ld_op(&Hs[(32 * tb + l32) * HP + 16 * ks + 8 * hh]);
        accY = mfma32(a, WdB[ks], accY);
      }
      const int o = 32 * ob + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * tb + 8 * (r >> 2) + 4 * hh + (r & 3);
        const float R = accY[r] - bf16_bits_to_f32(Vs[t * KP + o]);
        loss += R * R;
        dYs[t * KP + o] = f32_to_bf16_bits((2.0f / D) * R);
      }
    }
    __syncthreads();

    // 5. dH = dY W_d^T for this wave's hidden units; dG, dU.
    bf16x8 dGop[4], dUop[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16 accH = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = ld_op(&dYs[(32 * mt + l32) * KP + 16 * ks + 8 * hh]);
        accH = mfma32(a, WdTB[ks], accH);
      }
      float dg[16], du[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        du[r] = accH[r] * Aa[mt][r];
        dg[r] = accH[r] * GP[mt][r];
      }
      dGop[2 * mt] = pack8(&dg[0]);
      dGop[2 * mt + 1] = pack8(&dg[8]);
      dUop[2 * mt] = pack8(&du[0]);
      dUop[2 * mt + 1] = pack8(&du[8]);
    }

    // 6. Weight gradients; k-slot (hh, j) of k-step ks is token
    //    16ks + 8(j/4) + 4hh + j%4 (the register order of the C tiles above).
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      int trow[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) trow[j] = 16 * ks + 8 * (j >> 2) + 4 * hh + (j & 3);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        u32x4 q;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          q[j] = (uint32_t)dYs[trow[2 * j] * KP + 32 * nb + l32] |
                 ((uint32_t)dYs[trow[2 * j + 1] * KP + 32 * nb + l32] << 16);
        accWd[nb] = mfma32(Hop[ks], as_bf16x8(q), accWd[nb]);
      }
#pragma unroll
      for (int eb = 0; eb < 2; ++eb) {
        u32x4 q;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          q[j] = (uint32_t)Ks[trow[2 * j] * KP + 32 * eb + l32] |
                 ((uint32_t)Ks[trow[2 * j + 1] * KP + 32 * eb + l32] << 16);
        const bf16x8 a = as_bf16x8(q);
        accWg[eb] = mfma32(a, dGop[ks], accWg[eb]);
        accWu[eb] = mfma32(a, dUop[ks], accWu[eb]);
      }
    }
    __syncthreads();
  }

  // Partials in theta layout.
  float* out = part + ((int64_t)head * P + chunk) * PER_HEAD;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * hh + (r & 3);
      const int hid = 32 * w + row;        // gW_d rows
      const int o = 32 * b + l32;
      out[2 * DM + hid * D + o] = accWd[b][r];
      const int e = 32 * b + row;          // gW_g / gW_u rows
      const int hc = 32 * w + l32;
      out[e * M + hc] = accWg[b][r];
      out[DM + e * M + hc] = accWu[b][r];
    }
  }
  // Loss partial: fixed-order reduction (lanes, then waves).
  loss = wave_sum(loss);
  if (lane == 0) red[w] = loss;
  __syncthreads();
  if (tid == 0) loss_part[(int64_t)head * P + chunk] = ((red[0] + red[1]) + (red[2] + red[3])) * (1.0f / D);
}

// ---------------------------------------------------------------------------
// Read pass O = T(Q) per head. Tokens run across lanes here (MFMA columns),
// so the chain G^T = W_g^T Q^T -> H^T -> Y^T = W_d^T H^T contracts over e and
// then over hidden units with no transposes: each H^T tile is consumed from
// registers. Weights sit in LDS, pre-permuted to match the operand orders.
// Each wave handles 32 tokens per iteration.
// ---------------------------------------------------------------------------
constexpr int RT = 32;  // tokens per wave iteration

__global__ __launch_bounds__(256, 2) void read_bf16_kernel(const uint16_t* __restrict__ Q,
                                                           const float* __restrict__ theta,
                                                           uint16_t* __restrict__ O, int64_t n_tokens,
                                                           int n_heads, int P, int64_t n_blocks) {
  __shared__ __attribute__((aligned(16))) uint16_t WgP[M * KP];
  __shared__ __attribute__((aligned(16))) uint16_t WuP[M * KP];
  __shared__ __attribute__((aligned(16))) uint16_t WdP[D * HP];

  const int64_t blk = xcd_remap(blockIdx.x, n_blocks);
  const int head = (int)(blk / P);
  const int chunk = (int)(blk % P);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t C = (int64_t)n_heads * D;
  const float* th = theta + (int64_t)head * PER_HEAD;

  // A operand of G^T for k-step ks: lane (row hid, half hh) supplies
  // W_g[e = 32hh + 8ks + j][hid]; stored at WgP[hid][16ks + 8hh + j].
  for (int idx = tid; idx < M * D; idx += 256) {
    const int hid = idx / D, kk = idx % D;
    const int ks = kk >> 4, h2 = (kk >> 3) & 1, j = kk & 7;
    const int e = 32 * h2 + 8 * ks + j;
    WgP[hid * KP + kk] = f32_to_bf16_bits(th[e * M + hid]);
    WuP[hid * KP + kk] = f32_to_bf16_bits(th[DM + e * M + hid]);
  }
  // A operand of Y^T for k-step s: lane (row o, half hh) supplies
  // W_d[hid = 16s + 8(j/4) + 4hh + j%4][o] (the register order of H^T).
  for (int idx = tid; idx < D * M; idx += 256) {
    const int o = idx / M, kk = idx % M;
    const int s = kk >> 4, h2 = (kk >> 3) & 1, j = kk & 7;
    const int hid = 16 * s + 8 * (j >> 2) + 4 * h2 + (j & 3);
    WdP[o * HP + kk] = f32_to_bf16_bits(th[2 * DM + hid * D + o]);
  }
  __syncthreads();

  const int64_t n_tiles = (n_tokens + RT - 1) / RT;
  const int64_t tile_begin = n_tiles * chunk / P;
  const int64_t tile_end = n_tiles * (chunk + 1) / P;

  for (int64_t tile = tile_begin + w; tile < tile_end; tile += 4) {
    const int64_t t = tile * RT + l32;
    const bool valid = t < n_tokens;
    u32x4 qraw[4] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    if (valid) {
      const uint16_t* src = Q + t * C + (int64_t)head * D + 32 * hh;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qraw[ks] = ld16(src + 8 * ks);
    }
    bf16x8 q[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) q[ks] = as_bf16x8(qraw[ks]);
    f32x16 accY[2] = {f32x16{}, f32x16{}};
#pragma unroll 1
    for (int mt = 0; mt < 4; ++mt) {
      f32x16 g = f32x16{}, u = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int off = (32 * mt + l32) * KP + 16 * ks + 8 * hh;
        g = mfma32(ld_op(&WgP[off]), q[ks], g);
        u = mfma32(ld_op(&WuP[off]), q[ks], u);
      }
      float h[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float s = sigmoid_fast(g[r]);
        h[r] = g[r] * s * u[r];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 hop = pack8(&h[8 * half]);
        const int s = 2 * mt + half;
#pragma unroll
        for (int ot = 0; ot < 2; ++ot) {
          accY[ot] = mfma32(ld_op(&WdP[(32 * ot + l32) * HP + 16 * s + 8 * hh]), hop, accY[ot]);
        }
      }
    }
    if (valid) {
      uint16_t* dst = O + t * C + (int64_t)head * D;
#pragma unroll
      for (int ot = 0; ot < 2; ++ot) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 v;
          v[0] = pack_bf16x2(accY[ot][4 * q4 + 0], accY[ot][4 * q4 + 1]);
          v[1] = pack_bf16x2(accY[ot][4 * q4 + 2], accY[ot][4 * q4 + 3]);
          *reinterpret_cast<u32x2*>(dst + 32 * ot + 8 * q4 + 4 * hh) = v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_grad_partial_bf16(const void* K, const void* Vp, const float* theta, float* part,
                                    float* loss_part, int64_t n_tokens, int n_heads, int P,
                                    hipStream_t stream) {
  const int64_t n_blocks = (int64_t)n_heads * P;
  hipLaunchKernelGGL(grad_partial_bf16_kernel, dim3((unsigned)n_blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(Vp), theta, part,
                     loss_part, n_tokens, n_heads, P, n_blocks);
  return hipGetLastError();
}

hipError_t launch_read_bf16(const void* Q, const float* theta, void* O, int64_t n_tokens, int n_heads,
                            hipStream_t stream) {
  // Enough workgroups to fill 256 CUs twice over; each handles a contiguous
  // run of 32-token tiles of one head.
  const int64_t n_tiles = (n_tokens + RT - 1) / RT;
  int64_t P = (512 + n_heads - 1) / n_heads;
  if (P > n_tiles) P = n_tiles;
  if (P < 1) P = 1;
  const int64_t n_blocks = (int64_t)n_heads * P;
  hipLaunchKernelGGL(read_bf16_kernel, dim3((unsigned)n_blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(Q), theta, static_cast<uint16_t*>(O), n_tokens, n_heads,
                     (int)P, n_blocks);
  return hipGetLastError();
}

}  // namespace vggt3

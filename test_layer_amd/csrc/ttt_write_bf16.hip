// Write pass (bf16 MFMA): per-(head, token chunk) fp32 partials of the
// gradient of the inner loss, for the VGGT shape d = 64, m = 128.
//
// Fast-weight MLP per head (paper-graph summary "VGG-T3: Offline Feed-Forward
// 3D Reconstruction at Scale", section 3.4 "TTT MLP Architecture and Inner
// Optimization", bias-free SwiGLU):   T(x) = (silu(x W_g) * (x W_u)) W_d.
// Inner loss (Eq. 3 of that section with a squared error), per head:
//   L = sum_i (1/d) ||T(k_i) - v'_i||^2,
// whose gradient is a sum of per-token terms (Eq. 5, "Large-Scale Inference
// Strategies"); one workgroup sums a contiguous chunk of tokens of one head.
//
// Backward pass, with R = Y - V' and the factor 2/d (a power of two, so exact)
// applied once to the finished partials:
//   dH = R W_d^T, dU = dH * A, dG = dH * U silu'(G),
//   gW_d += H^T R,  gW_g += K^T dG,  gW_u += K^T dU.
// R is never rounded as a whole: Y (tiny next to V') would vanish in a bf16
// R. Instead Y is rounded to bf16 on its own and -V' (exact in bf16) enters
// the R contractions as a second MFMA operand, so no information is lost.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16): a C tile keeps rows in registers and
// columns across lanes, and is reused as an operand of any contraction over
// its rows. Tokens are the rows of G, U, Y, dH, so H, dG and dU feed the
// weight-gradient contractions (over tokens) straight from registers. The
// remaining operand orders come from LDS, with ds_read_b64_tr_b16 transposing
// 4x16 blocks on the way into registers.
//
// Workgroup = 4 waves; wave w owns hidden units [32w, 32w+32): G, U, H, dH,
// dG, dU for those units and the matching gradient slices gW_g[:, w-slice],
// gW_u[:, w-slice], gW_d[w-slice, :] (96 fp32 accumulators per lane, kept for
// the whole chunk). W_g / W_u operands live in registers, W_d in LDS. Per
// 64-token tile c the workgroup runs
//   B0 | G,U(c) ; gradients(c-1) ; SwiGLU(c) -> H ; stage K,V'(c+1)
//   B1 | Y(c) = H W_d ; R, loss ; Y -> LDS
//   B2 | dH(c) = (Y - V') W_d^T ; dG, dU
// so the gradient MFMAs of one tile overlap the SwiGLU VALU work of the next.
// K and V' tiles rotate through 3 LDS buffers and Y through 2; global loads of
// tile c+2 are issued while tile c computes. All LDS addressing is 32-bit.
#include "bf16_ops.hpp"
#include "kernels.hpp"

#ifndef VGGT3_WRITE_TP
#define VGGT3_WRITE_TP 72
#endif
#ifndef VGGT3_WRITE_HP
#define VGGT3_WRITE_HP 72
#endif
#ifndef VGGT3_WRITE_WP
#define VGGT3_WRITE_WP 72
#endif

namespace vggt3 {
namespace {

constexpr int D = 64;      // inputs / outputs of T per head
constexpr int M = 128;     // hidden units
constexpr int T = 64;      // tokens per tile
constexpr int DM = D * M;
constexpr int PER_HEAD = 3 * DM;
constexpr int TP = VGGT3_WRITE_TP;   // pitch (elements) of [64][64] tiles: K[t][e], Vn[t][o], Y[o][t]
constexpr int HPT = VGGT3_WRITE_HP;  // pitch of H[hid][t]
constexpr int WP = VGGT3_WRITE_WP;   // pitch of W_d[hid][o]
constexpr int KV_BUFS = 3;
constexpr int Y_BUFS = 2;
constexpr int TSZ = T * TP;          // elements per token tile

// LDS map (elements of bf16).
constexpr int OFF_K = 0;
constexpr int OFF_V = OFF_K + KV_BUFS * TSZ;
constexpr int OFF_Y = OFF_V + KV_BUFS * TSZ;
constexpr int OFF_H = OFF_Y + Y_BUFS * TSZ;
constexpr int OFF_W = OFF_H + M * HPT;
constexpr int LDS_ELEMS = OFF_W + M * WP;

typedef __attribute__((address_space(3))) uint16_t lu16;
typedef __attribute__((address_space(3))) u32x4 lu32x4;
typedef __attribute__((address_space(3))) u32x2 lu32x2;

__device__ __forceinline__ u32x4 lld16(const lu16* p) { return *(const lu32x4*)p; }
__device__ __forceinline__ u32x2 lld8(const lu16* p) { return *(const lu32x2*)p; }
__device__ __forceinline__ void lst16(lu16* p, const u32x4& v) { *(lu32x4*)p = v; }
__device__ __forceinline__ void lst8(lu16* p, const u32x2& v) { *(lu32x2*)p = v; }
__device__ __forceinline__ u32x2 ltr(const lu16* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}
__device__ __forceinline__ bf16x8 lop(const lu16* p) { return as_bf16x8(lld16(p)); }
__device__ __forceinline__ bf16x8 ltr_op(const lu16* p0, const lu16* p1) {
  const u32x2 a = ltr(p0), b = ltr(p1);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}
__device__ __forceinline__ bf16x8 lpair_op(const lu16* p0, const lu16* p1) {
  const u32x2 a = lld8(p0), b = lld8(p1);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

// Keeps a value in accumulation registers: MFMA reads its A/B operands from
// them directly, which leaves the architectural VGPRs for in-flight LDS data.
#ifndef VGGT3_PIN_AGPR
#define VGGT3_PIN_AGPR 1
#endif
__device__ __forceinline__ void to_agpr(bf16x8& v) {
#if VGGT3_PIN_AGPR
  asm volatile("" : "+a"(v));
#endif
}

__global__ __launch_bounds__(256, 1) void grad_partial_bf16_kernel(
    const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg, const float* __restrict__ theta,
    float* __restrict__ part, float* __restrict__ loss_part, int64_t n_tokens, int n_heads, int P,
    int64_t n_blocks) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[LDS_ELEMS];
  __shared__ float red[4];
  lu16* const lds = (lu16*)smem;

  const int64_t blk = xcd_remap(blockIdx.x, n_blocks);
  const int head = (int)(blk / P);
  const int chunk = (int)(blk % P);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;               // k-half of a 32x32x16 operand
  const int cb = 16 * ((lane >> 4) & 1);  // column base of this lane's 16-lane group
  const int jr = (lane & 15) >> 2;        // transpose-read source row within the group
  const int q4 = lane & 3;                // transpose-read source column quad
  const int64_t C = (int64_t)n_heads * D;
  const int tb = w >> 1, ob = w & 1;      // this wave's Y tile (tokens 32tb.., outputs 32ob..)

  const float* th = theta + (int64_t)head * PER_HEAD;
  const float* Wg = th;
  const float* Wu = th + DM;
  const float* Wd = th + 2 * DM;

  // W_g / W_u operands in registers: B[k = e][j = hid], e = 16ks + 8hh + jj, hid = 32w + l32.
  bf16x8 WgB[4], WuB[4];
  {
    const int hid = 32 * w + l32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float g[8], u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = 16 * ks + 8 * hh + j;
        g[j] = Wg[e * M + hid];
        u[j] = Wu[e * M + hid];
      }
      WgB[ks] = pack8(g);
      WuB[ks] = pack8(u);
      to_agpr(WgB[ks]);
      to_agpr(WuB[ks]);
    }
  }
  // W_d (bf16) in LDS, natural [hid][o] layout.
  for (int idx = tid; idx < M * D / 2; idx += 256) {
    const int hid = (2 * idx) / D, o = (2 * idx) % D;
    *(__attribute__((address_space(3))) uint32_t*)(lds + OFF_W + hid * WP + o) =
        pack_bf16x2(Wd[hid * D + o], Wd[hid * D + o + 1]);
  }

  f32x16 accWd[2], accWg[2], accWu[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    accWd[i] = f32x16{};
    accWg[i] = f32x16{};
    accWu[i] = f32x16{};
  }
  float loss = 0.0f;

  const int64_t n_tiles_all = (n_tokens + T - 1) / T;
  const int64_t tile_begin = n_tiles_all * chunk / P;
  const int nt = (int)(n_tiles_all * (chunk + 1) / P - tile_begin);

  // Lane-constant LDS offsets (elements).
  const int o_row = l32 * TP + 8 * hh;                    // row-major operand rows (b128)
  const int o_tr = (4 * hh + jr) * TP + cb + 4 * q4;       // transpose reads over token rows
  const int o_htr = (8 * hh + jr) * HPT + cb + 4 * q4;     // transpose reads of H[hid][t]
  const int o_ytr = (8 * hh + jr) * TP + cb + 4 * q4;      // transpose reads of Y[o][t]
  const int o_wtr = (8 * hh + jr) * WP + cb + 4 * q4;      // transpose reads of W_d[hid][o]
  const int o_wrow = (32 * w + l32) * WP + 8 * hh;         // W_d rows of this wave's units
  const int o_yrow = l32 * TP + 4 * hh;                    // Y[o][t] runs for gW_d
  const int o_hst = (32 * w + l32) * HPT + 4 * hh;         // H stores
  const int o_yst = (32 * ob + l32) * TP + 32 * tb + 4 * hh;  // Y stores

  // Tile staging: thread -> rows (tid>>3) and (tid>>3)+32, 8 channels at (tid&7)*8.
  // Loads are unconditional (rows past the end re-read the last token and are
  // zeroed), which keeps the compiler's load-counter waits exact.
  const int srow = tid >> 3, scol = (tid & 7) * 8;
  const int o_stage = srow * TP + scol;
  const uint16_t* Kh = Kg + (int64_t)head * D + scol;
  const uint16_t* Vh = Vg + (int64_t)head * D + scol;
  u32x4 kr[2], vr[2];
  auto load_tile = [&](int i) {
    const int64_t tok0 = (tile_begin + i) * T;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      int64_t tok = tok0 + srow + 32 * s;
      tok = tok < n_tokens ? tok : n_tokens - 1;
      kr[s] = ld16(Kh + tok * C);
      vr[s] = ld16(Vh + tok * C);
    }
  };
  auto store_tile = [&](int i) {
    const int buf = i % KV_BUFS;
    const int64_t tok0 = (tile_begin + i) * T;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bool ok = tok0 + srow + 32 * s < n_tokens;
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      lst16(lds + OFF_K + buf * TSZ + o_stage + 32 * s * TP, ok ? kr[s] : z);
      lst16(lds + OFF_V + buf * TSZ + o_stage + 32 * s * TP,
            ok ? (vr[s] ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u}) : z);
    }
  };

  // Operands of the previous tile's gradient contractions (k-slot jj of k-step
  // ks is token 16ks + 8(jj/4) + 4hh + jj%4, the register order of C tiles).
  // They start at zero, with zeroed "tile -1" buffers, so the gradient step
  // runs unconditionally inside the loop body and adds nothing the first time.
  bf16x8 Hop[4], dGop[4], dUop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    Hop[ks] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    dGop[ks] = Hop[ks];
    dUop[ks] = Hop[ks];
  }
  for (int idx = tid * 8; idx < TSZ; idx += 256 * 8) {
    lst16(lds + OFF_K + (KV_BUFS - 1) * TSZ + idx, u32x4{0u, 0u, 0u, 0u});
    lst16(lds + OFF_V + (KV_BUFS - 1) * TSZ + idx, u32x4{0u, 0u, 0u, 0u});
    lst16(lds + OFF_Y + (Y_BUFS - 1) * TSZ + idx, u32x4{0u, 0u, 0u, 0u});
  }

  auto gradients = [&](int kvb, int yb) {
    const lu16* Kp = lds + OFF_K + kvb * TSZ;
    const lu16* Vp = lds + OFF_V + kvb * TSZ;
    const lu16* Yp = lds + OFF_Y + yb * TSZ;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const lu16* yr = Yp + o_yrow + 32 * nb * TP + 16 * ks;
        const bf16x8 yB = lpair_op(yr, yr + 8);
        const lu16* vt = Vp + o_tr + 16 * ks * TP + 32 * nb;
        const bf16x8 vB = ltr_op(vt, vt + 8 * TP);
        accWd[nb] = mfma32(Hop[ks], yB, accWd[nb]);
        accWd[nb] = mfma32(Hop[ks], vB, accWd[nb]);
      }
#pragma unroll
      for (int eb = 0; eb < 2; ++eb) {
        const lu16* kt = Kp + o_tr + 16 * ks * TP + 32 * eb;
        const bf16x8 kA = ltr_op(kt, kt + 8 * TP);
        accWg[eb] = mfma32(kA, dGop[ks], accWg[eb]);
        accWu[eb] = mfma32(kA, dUop[ks], accWu[eb]);
      }
    }
  };

  if (nt > 0) {
    load_tile(0);
    store_tile(0);
    if (nt > 1) load_tile(1);
  }

  for (int i = 0; i < nt; ++i) {
    const int kvb = i % KV_BUFS;
    const int yb = i & 1;
    const lu16* Kc = lds + OFF_K + kvb * TSZ;
    const lu16* Vc = lds + OFF_V + kvb * TSZ;
    lu16* Yc = lds + OFF_Y + yb * TSZ;
    __syncthreads();  // B0: K, V'(i) staged; everything of tile i-2 consumed

    // G, U of tile i: element (mt, r) is token 32mt + 8(r/4) + 4hh + r%4, unit 32w + l32.
    f32x16 accG[2], accU[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      accG[mt] = f32x16{};
      accU[mt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = lop(Kc + o_row + 32 * mt * TP + 16 * ks);
        accG[mt] = mfma32(a, WgB[ks], accG[mt]);
        accU[mt] = mfma32(a, WuB[ks], accU[mt]);
      }
    }

    gradients((i + KV_BUFS - 1) % KV_BUFS, (i + 1) & 1);  // tile i-1

    // SwiGLU: s = sigmoid(G), A = G s, H = A U, gp = U silu'(G) = U s + H (1 - s).
    // A and gp are kept as bf16 pairs until the backward step.
    uint32_t Ap[2][8], GPp[2][8];
    float Hf[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float a2[2], gp2[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float g = accG[mt][r + k];
          const float u = accU[mt][r + k];
          const float s = sigmoid_fast(g);
          const float a = g * s;
          const float h = a * u;
          a2[k] = a;
          Hf[mt][r + k] = h;
          gp2[k] = fmaf(-h, s, fmaf(u, s, h));
        }
        Ap[mt][r / 2] = pack_bf16x2(a2[0], a2[1]);
        GPp[mt][r / 2] = pack_bf16x2(gp2[0], gp2[1]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      Hop[ks] = pack8(&Hf[ks >> 1][8 * (ks & 1)]);
      const u32x4 hv = as_u32x4(Hop[ks]);
      lu16* hp = lds + OFF_H + o_hst + 32 * (ks >> 1) + 16 * (ks & 1);
      lst8(hp, u32x2{hv[0], hv[1]});
      lst8(hp + 8, u32x2{hv[2], hv[3]});
    }
    // Stage tile i+1 (loaded during the previous tile) and start loading i+2.
    if (i + 1 < nt) {
      store_tile(i + 1);
      if (i + 2 < nt) load_tile(i + 2);
    }
    __syncthreads();  // B1: H(i) complete

    // Y tile (tokens 32tb.., outputs 32ob..) = H W_d; R = Y - V'; Y -> LDS [o][t].
    {
      f32x16 accY = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const lu16* hp = lds + OFF_H + o_htr + 16 * ks * HPT + 32 * tb;
        const lu16* wp = lds + OFF_W + o_wtr + 16 * ks * WP + 32 * ob;
        accY = mfma32(ltr_op(hp, hp + 4 * HPT), ltr_op(wp, wp + 4 * WP), accY);
      }
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const u32x2 vn = ltr(Vc + o_tr + (32 * tb + 8 * rg) * TP + 32 * ob);
        const float r0 = accY[4 * rg + 0] + bf16_lo(vn[0]);
        const float r1 = accY[4 * rg + 1] + bf16_hi(vn[0]);
        const float r2 = accY[4 * rg + 2] + bf16_lo(vn[1]);
        const float r3 = accY[4 * rg + 3] + bf16_hi(vn[1]);
        loss = fmaf(r0, r0, loss);
        loss = fmaf(r1, r1, loss);
        loss = fmaf(r2, r2, loss);
        loss = fmaf(r3, r3, loss);
        lst8(Yc + o_yst + 8 * rg, u32x2{pack_bf16x2(accY[4 * rg + 0], accY[4 * rg + 1]),
                                        pack_bf16x2(accY[4 * rg + 2], accY[4 * rg + 3])});
      }
    }
    __syncthreads();  // B2: Y(i) complete

    // dH = (Y - V') W_d^T for this wave's hidden units; dU = dH A, dG = dH gp.
    {
      bf16x8 WdT[4];  // B[k = o][j = hid], o = 16ks + 8hh + jj, hid = 32w + l32
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) WdT[ks] = lop(lds + OFF_W + o_wrow + 16 * ks);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x16 accH = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const lu16* yp = Yc + o_ytr + 16 * ks * TP + 32 * mt;
          accH = mfma32(ltr_op(yp, yp + 4 * TP), WdT[ks], accH);
          accH = mfma32(lop(Vc + o_row + 32 * mt * TP + 16 * ks), WdT[ks], accH);
        }
        float dg[16], du[16];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          du[r] = accH[r] * bf16_lo(Ap[mt][r / 2]);
          du[r + 1] = accH[r + 1] * bf16_hi(Ap[mt][r / 2]);
          dg[r] = accH[r] * bf16_lo(GPp[mt][r / 2]);
          dg[r + 1] = accH[r + 1] * bf16_hi(GPp[mt][r / 2]);
        }
        dGop[2 * mt] = pack8(&dg[0]);
        dGop[2 * mt + 1] = pack8(&dg[8]);
        dUop[2 * mt] = pack8(&du[0]);
        dUop[2 * mt + 1] = pack8(&du[8]);
        to_agpr(dGop[2 * mt]);
        to_agpr(dGop[2 * mt + 1]);
        to_agpr(dUop[2 * mt]);
        to_agpr(dUop[2 * mt + 1]);
      }
    }
  }
  if (nt > 0) gradients((nt - 1) % KV_BUFS, (nt - 1) & 1);

  // Partials in theta layout, times 2/d.
  constexpr float kScale = 2.0f / D;
  float* out = part + ((int64_t)head * P + chunk) * PER_HEAD;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * hh + (r & 3);
      const int hid = 32 * w + row;  // gW_d rows
      const int o = 32 * b + l32;
      out[2 * DM + hid * D + o] = accWd[b][r] * kScale;
      const int e = 32 * b + row;    // gW_g / gW_u rows
      const int hc = 32 * w + l32;
      out[e * M + hc] = accWg[b][r] * kScale;
      out[DM + e * M + hc] = accWu[b][r] * kScale;
    }
  }
  loss = wave_sum(loss);
  if (lane == 0) red[w] = loss;
  __syncthreads();
  if (tid == 0)
    loss_part[(int64_t)head * P + chunk] = ((red[0] + red[1]) + (red[2] + red[3])) * (1.0f / D);
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

}  // namespace vggt3

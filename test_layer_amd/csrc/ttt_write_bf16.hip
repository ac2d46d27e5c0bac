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
// gW_u[:, w-slice], gW_d[w-slice, :] (96 fp32 accumulators per lane, kept in
// registers for the whole chunk). Per 64-token tile c the workgroup runs
//   B0 | G,U(c) ; gradients(c-1) ; SwiGLU(c) -> H ; stage K,V'(c+1)
//   B1 | Y(c) = H W_d ; R, loss ; Y -> LDS
//   B2 | dH(c) = (Y - V') W_d^T ; dG, dU
// so the gradient MFMAs of one tile overlap the SwiGLU VALU work of the next.
// K and V' tiles rotate through 3 LDS buffers and Y through 2; global loads of
// tile c+2 are issued while tile c computes.
#include "bf16_ops.hpp"
#include "kernels.hpp"

namespace vggt3 {
namespace {

constexpr int D = 64;      // inputs / outputs of T per head
constexpr int M = 128;     // hidden units
constexpr int T = 64;      // tokens per tile
constexpr int DM = D * M;
constexpr int PER_HEAD = 3 * DM;
constexpr int TP = 72;     // LDS pitch (elements) of [64][64] tiles: K[t][e], Vn[t][o], Y[o][t]
constexpr int HPT = 72;    // LDS pitch of H[hid][t]
constexpr int KV_BUFS = 3;
constexpr int Y_BUFS = 2;

struct Smem {
  uint16_t K[KV_BUFS][T * TP];
  uint16_t Vn[KV_BUFS][T * TP];  // -V'
  uint16_t Y[Y_BUFS][D * TP];    // [o][t]
  uint16_t H[M * HPT];           // [hid][t]
  float red[4];
};

__global__ __launch_bounds__(256, 1) void grad_partial_bf16_kernel(
    const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg, const float* __restrict__ theta,
    float* __restrict__ part, float* __restrict__ loss_part, int64_t n_tokens, int n_heads, int P,
    int64_t n_blocks) {
  __shared__ __attribute__((aligned(16))) Smem sm;

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

  // Weight operands (bf16, round to nearest even) held in registers.
  //   WgB/WuB[ks]: B[k = e][j = hid], e = 16ks + 8hh + jj, hid = 32w + l32   (G, U)
  //   WdB[ks]:     B[k = hid][j = o], hid = 16ks + 8hh + jj, o = 32ob + l32  (Y)
  //   WdTB[ks]:    B[k = o][j = hid], o = 16ks + 8hh + jj, hid = 32w + l32   (dH)
  bf16x8 WgB[4], WuB[4], WdB[8], WdTB[4];
  {
    const int hid = 32 * w + l32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float g[8], u[8], dt[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = 16 * ks + 8 * hh + j;
        g[j] = Wg[e * M + hid];
        u[j] = Wu[e * M + hid];
        dt[j] = Wd[hid * D + e];
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

  const int64_t n_tiles_all = (n_tokens + T - 1) / T;
  const int64_t tile_begin = n_tiles_all * chunk / P;
  const int nt = (int)(n_tiles_all * (chunk + 1) / P - tile_begin);

  // Tile staging: thread -> rows (tid>>3) and (tid>>3)+32, 8 channels at (tid&7)*8.
  const int srow = tid >> 3, scol = (tid & 7) * 8;
  const uint16_t* Kh = Kg + (int64_t)head * D + scol;
  const uint16_t* Vh = Vg + (int64_t)head * D + scol;
  u32x4 kr[2], vr[2];
  auto load_tile = [&](int i) {
    const int64_t tok0 = (tile_begin + i) * T;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t tok = tok0 + srow + 32 * s;
      kr[s] = u32x4{0u, 0u, 0u, 0u};
      vr[s] = u32x4{0u, 0u, 0u, 0u};
      if (tok < n_tokens) {
        kr[s] = ld16(Kh + tok * C);
        vr[s] = ld16(Vh + tok * C);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int r = srow + 32 * s;
      st16(&sm.K[buf][r * TP + scol], kr[s]);
      st16(&sm.Vn[buf][r * TP + scol], vr[s] ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u});
    }
  };

  // Operands of the previous tile's gradient contractions (k-slot jj of k-step
  // ks is token 16ks + 8(jj/4) + 4hh + jj%4, the register order of C tiles).
  // They start at zero, with zeroed "tile -1" buffers, so that the gradient
  // step can run unconditionally inside the loop body (one basic block for the
  // MFMA / VALU overlap) and contributes nothing on the first iteration.
  bf16x8 Hop[4], dGop[4], dUop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    Hop[ks] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    dGop[ks] = Hop[ks];
    dUop[ks] = Hop[ks];
  }
  for (int idx = tid * 8; idx < T * TP; idx += 256 * 8) {
    st16(&sm.K[KV_BUFS - 1][idx], u32x4{0u, 0u, 0u, 0u});
    st16(&sm.Vn[KV_BUFS - 1][idx], u32x4{0u, 0u, 0u, 0u});
    st16(&sm.Y[Y_BUFS - 1][idx], u32x4{0u, 0u, 0u, 0u});
  }

  auto gradients = [&](int kvb, int yb) {
    const uint16_t* Kp = sm.K[kvb];
    const uint16_t* Vp = sm.Vn[kvb];
    const uint16_t* Yp = sm.Y[yb];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int r0 = 16 * ks + 4 * hh + jr;  // transpose-read source rows (tokens)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int o = 32 * nb + l32;
        const bf16x8 yB = pair_op(&Yp[o * TP + 16 * ks + 4 * hh], &Yp[o * TP + 16 * ks + 8 + 4 * hh]);
        const int oc = 32 * nb + cb + 4 * q4;
        const bf16x8 vB = tr_op(&Vp[r0 * TP + oc], &Vp[(r0 + 8) * TP + oc]);
        accWd[nb] = mfma32(Hop[ks], yB, accWd[nb]);
        accWd[nb] = mfma32(Hop[ks], vB, accWd[nb]);
      }
#pragma unroll
      for (int eb = 0; eb < 2; ++eb) {
        const int ec = 32 * eb + cb + 4 * q4;
        const bf16x8 kA = tr_op(&Kp[r0 * TP + ec], &Kp[(r0 + 8) * TP + ec]);
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
    const uint16_t* Kc = sm.K[kvb];
    const uint16_t* Vc = sm.Vn[kvb];
    __syncthreads();  // B0: K, V'(i) staged; everything of tile i-2 consumed

    // G, U of tile i: element (mt, r) is token 32mt + 8(r/4) + 4hh + r%4, unit 32w + l32.
    f32x16 accG[2], accU[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      accG[mt] = f32x16{};
      accU[mt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = ld_op(&Kc[(32 * mt + l32) * TP + 16 * ks + 8 * hh]);
        accG[mt] = mfma32(a, WgB[ks], accG[mt]);
        accU[mt] = mfma32(a, WuB[ks], accU[mt]);
      }
    }

    gradients((i + KV_BUFS - 1) % KV_BUFS, (i + 1) & 1);  // tile i-1

    // SwiGLU: s = sigmoid(G), A = G s, H = A U, gp = U silu'(G) = U s + H (1 - s).
    float Af[2][16], GP[2][16], Hf[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float g = accG[mt][r];
        const float u = accU[mt][r];
        const float s = sigmoid_fast(g);
        const float a = g * s;
        const float h = a * u;
        Af[mt][r] = a;
        Hf[mt][r] = h;
        GP[mt][r] = fmaf(-h, s, fmaf(u, s, h));
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Hop[ks] = pack8(&Hf[ks >> 1][8 * (ks & 1)]);
    {
      const int hid = 32 * w + l32;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 hv = as_u32x4(Hop[ks]);
        const int t0 = 32 * (ks >> 1) + 16 * (ks & 1) + 4 * hh;
        st8(&sm.H[hid * HPT + t0], u32x2{hv[0], hv[1]});
        st8(&sm.H[hid * HPT + t0 + 8], u32x2{hv[2], hv[3]});
      }
    }
    // Stage tile i+1 (loaded during the previous tile) and start loading i+2.
    if (i + 1 < nt) {
      store_tile((i + 1) % KV_BUFS);
      if (i + 2 < nt) load_tile(i + 2);
    }
    __syncthreads();  // B1: H(i) complete

    // Y tile (tokens 32tb.., outputs 32ob..) = H W_d; R = Y - V'; Y -> LDS [o][t].
    {
      f32x16 accY = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int hr = 16 * ks + 8 * hh + jr;
        const int tc = 32 * tb + cb + 4 * q4;
        const bf16x8 a = tr_op(&sm.H[hr * HPT + tc], &sm.H[(hr + 4) * HPT + tc]);
        accY = mfma32(a, WdB[ks], accY);
      }
      const int o = 32 * ob + l32;
      uint16_t* Yc = sm.Y[yb];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int t0 = 32 * tb + 8 * rg + 4 * hh;
        const u32x2 vn = lds_tr16(&Vc[(t0 + jr) * TP + 32 * ob + cb + 4 * q4]);
        const float r0 = accY[4 * rg + 0] + bf16_lo(vn[0]);
        const float r1 = accY[4 * rg + 1] + bf16_hi(vn[0]);
        const float r2 = accY[4 * rg + 2] + bf16_lo(vn[1]);
        const float r3 = accY[4 * rg + 3] + bf16_hi(vn[1]);
        loss = fmaf(r0, r0, loss);
        loss = fmaf(r1, r1, loss);
        loss = fmaf(r2, r2, loss);
        loss = fmaf(r3, r3, loss);
        st8(&Yc[o * TP + t0], u32x2{pack_bf16x2(accY[4 * rg + 0], accY[4 * rg + 1]),
                                    pack_bf16x2(accY[4 * rg + 2], accY[4 * rg + 3])});
      }
    }
    __syncthreads();  // B2: Y(i) complete

    // dH = (Y - V') W_d^T for this wave's hidden units; dU = dH A, dG = dH gp.
    {
      const uint16_t* Yc = sm.Y[yb];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x16 accH = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int orow = 16 * ks + 8 * hh + jr;
          const int tc = 32 * mt + cb + 4 * q4;
          const bf16x8 ya = tr_op(&Yc[orow * TP + tc], &Yc[(orow + 4) * TP + tc]);
          const bf16x8 va = ld_op(&Vc[(32 * mt + l32) * TP + 16 * ks + 8 * hh]);
          accH = mfma32(ya, WdTB[ks], accH);
          accH = mfma32(va, WdTB[ks], accH);
        }
        float dg[16], du[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          du[r] = accH[r] * Af[mt][r];
          dg[r] = accH[r] * GP[mt][r];
        }
        dGop[2 * mt] = pack8(&dg[0]);
        dGop[2 * mt + 1] = pack8(&dg[8]);
        dUop[2 * mt] = pack8(&du[0]);
        dUop[2 * mt + 1] = pack8(&du[8]);
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
  if (lane == 0) sm.red[w] = loss;
  __syncthreads();
  if (tid == 0)
    loss_part[(int64_t)head * P + chunk] = ((sm.red[0] + sm.red[1]) + (sm.red[2] + sm.red[3])) * (1.0f / D);
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

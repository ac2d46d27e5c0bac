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
// its rows. Tokens are the rows of G, U, dH, so H, dG and dU feed the
// weight-gradient contractions (over tokens) straight from registers. The
// remaining operand orders come from LDS, with ds_read_b64_tr_b16 transposing
// 4x16 blocks on the way into registers.
//
// Workgroup = 4 waves; wave w owns hidden units [32w, 32w+32): G, U, H, dH,
// dG, dU for those units and the matching gradient slices gW_g[:, w-slice],
// gW_u[:, w-slice], gW_d[w-slice, :] (96 fp32 accumulators per lane, kept for
// the whole chunk). W_g / W_u operands live in registers, W_d in LDS twice:
// [hid][o] for dH, and [o][hid] so that the Y phase reads its operand with
// plain 16-byte loads (transposing LDS reads cost about twice as much). Per
// 32-token tile c the workgroup runs
//   B0 | G,U(c) ; SwiGLU(c) -> H ; stage K,V'(c+1), load c+3
//   B1 | Y(c) = H W_d (16x16x32 MFMA tiles over all hidden units) ; loss ; Y -> LDS [o][t]
//   B2 | dH(c) = (Y - V') W_d^T ; dG, dU ; gW_d, gW_g, gW_u += tile c
// With the dot-product loss L = -sum_i T(k_i) . v'_i ("The dot product loss",
// same section), dL/dY = -V' does not depend on Y: the Y phase and its two
// barriers drop out, dH = -V' W_d^T, gW_d += H^T (-V'), and the loss is
// sum H * dH over the tile (= -sum Y . V').
// The loss value is a diagnostic: with LOSS false (the caller asked for no
// loss) the residual R = Y - V' is never formed (the gradient uses Y and -V'
// as separate operands anyway), and the loss partial is written as NaN.
// The kernel is sized (about 67 KB of LDS, at most 256 registers per lane, all
// of them architectural VGPRs, so MFMA results need no copies before VALU use)
// so that two workgroups share a CU: while one waits at a barrier or on LDS,
// the other's MFMA and VALU work fills the SIMDs. All LDS addressing is 32-bit.
#include "bf16_ops.hpp"
#include "kernels.hpp"

#ifndef VGGT3_WRITE_TP
#define VGGT3_WRITE_TP 72
#endif
#ifndef VGGT3_WRITE_HP
#define VGGT3_WRITE_HP 36
#endif
#ifndef VGGT3_WRITE_WP
#define VGGT3_WRITE_WP 72
#endif

namespace vggt3 {
namespace {

constexpr int D = 64;      // inputs / outputs of T per head
constexpr int M = 128;     // hidden units
constexpr int T = 32;      // tokens per tile
static_assert(T == kGradTileBf16, "the chunking cuts tokens in units of this tile");
constexpr int DM = D * M;
constexpr int PER_HEAD = 3 * DM;
constexpr int TP = VGGT3_WRITE_TP;   // pitch (elements) of [32][64] token tiles: K, -V' ([t][ch])
constexpr int HPT = VGGT3_WRITE_HP;  // pitch of H[hid][t]
constexpr int WP = VGGT3_WRITE_WP;   // pitch of W_d[hid][o]
constexpr int YP = 36;               // pitch of Y[o][t]: a lane stores its 4 tokens of one output at once
constexpr int KV_BUFS = 2;
constexpr int TSZ = T * TP;          // elements per token tile

// LDS map (elements of bf16).
constexpr int OFF_K = 0;
constexpr int OFF_V = OFF_K + KV_BUFS * TSZ;
constexpr int OFF_Y = OFF_V + KV_BUFS * TSZ;
constexpr int OFF_H = OFF_Y + TSZ;
constexpr int OFF_W = OFF_H + M * HPT;
constexpr int WTP = M + 8;             // pitch of W_d^T[o][hid]
constexpr int OFF_WT = OFF_W + M * WP;
constexpr int LDS_ELEMS = OFF_WT + D * WTP;
static_assert(LDS_ELEMS * 2 <= 80 * 1024, "two workgroups per CU");
static_assert(64 * YP <= TSZ, "Y tile");

typedef __attribute__((address_space(3))) uint16_t lu16;
typedef __attribute__((address_space(3))) u32x4 lu32x4;
typedef __attribute__((address_space(3))) u32x2 lu32x2;

__device__ __forceinline__ u32x4 lld16(const lu16* p) { return *(const lu32x4*)p; }
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

// 16x16x32 bf16 MFMA, fp32 accumulate.
//   A operand: lane l holds A[row = l%16][k = 8*(l/16) + j], j = 0..7
//   B operand: lane l holds B[k = 8*(l/16) + j][col = l%16]
//   C/D:       lane l, register r holds C[row = 4*(l/16) + r][col = l%16]
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <bool DOT, bool LOSS>
__global__ __launch_bounds__(256, 2) void grad_partial_bf16_kernel(
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
  const int g4 = lane >> 4;               // k-quarter of a 16x16x32 operand
  const int i16 = lane & 15;
  const int cb = 16 * ((lane >> 4) & 1);  // column base of this lane's 16-lane group (32-wide reads)
  const int jr = (lane & 15) >> 2;        // transpose-read source row within the group
  const int q4 = lane & 3;                // transpose-read source column quad
  const int64_t C = (int64_t)n_heads * D;
  const int tb = w >> 1;                  // this wave's Y rows: tokens 16tb..16tb+15
  const int ob = 2 * (w & 1);             // and Y column blocks ob, ob+1 (16 outputs each)

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
    }
  }
  // W_d (bf16) in LDS, natural [hid][o] layout.
  for (int idx = tid; idx < M * D / 2; idx += 256) {
    const int hid = (2 * idx) / D, o = (2 * idx) % D;
    *(__attribute__((address_space(3))) uint32_t*)(lds + OFF_W + hid * WP + o) =
        pack_bf16x2(Wd[hid * D + o], Wd[hid * D + o + 1]);
  }
  // and transposed, [o][hid], for the Y phase's B operand.
  if (!DOT) {
    for (int idx = tid; idx < M * D / 2; idx += 256) {
      const int o = (2 * idx) / M, hid = (2 * idx) % M;
      *(__attribute__((address_space(3))) uint32_t*)(lds + OFF_WT + o * WTP + hid) =
          pack_bf16x2(Wd[hid * D + o], Wd[(hid + 1) * D + o]);
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

  // Lane-constant LDS offsets (elements).
  const int o_row = l32 * TP + 8 * hh;                     // token-row operand reads (b128)
  const int o_tr = (4 * hh + jr) * TP + cb + 4 * q4;        // transpose reads over token rows
  const int o_hst = (32 * w + l32) * HPT + 4 * hh;          // H stores
  const int o_ha = (8 * g4 + jr) * HPT + 16 * tb + 4 * q4;  // Y phase: H^T reads (A operand)
  const int o_wtb = (16 * ob + i16) * WTP + 8 * g4;         // Y phase: W_d^T reads (B operand)
  const int o_vl = (16 * tb + 4 * g4 + jr) * TP + 16 * ob + 4 * q4;  // Y phase: -V' at the C positions
  const int o_yst = (16 * ob + i16) * YP + 16 * tb + 4 * g4;         // Y stores: 4 tokens of one output
  const int o_ytr = (8 * hh + jr) * YP + cb + 4 * q4;                // dH phase: Y^T transpose reads
  const int o_wrow = (32 * w + l32) * WP + 8 * hh;          // W_d rows of this wave's units

  // Tile staging: thread -> row tid>>3, 8 channels at (tid&7)*8. K and V'
  // are read through buffer descriptors built per tile from 64-bit scalar
  // arithmetic: based at the tile's first token and this head, with a range
  // that ends at the tensor's end. The lane offset is fixed; rows at or past
  // n_tokens lie beyond the range and read as zeros, which also keeps the loads
  // unconditional, so the compiler's load-counter waits stay exact.
  const int srow = tid >> 3, scol = (tid & 7) * 8;
  const int o_stage = srow * TP + scol;
  const int lane_off = (srow * (int)C + scol) * 2;
  auto load_tile = [&](int i, u32x4& kr, u32x4& vr) {
    const int64_t t0 = (tile_begin + i) * T;
    const int64_t off = t0 * C + (int64_t)head * D;
    const int64_t range = (n_tokens - t0) * C * 2 - (int64_t)head * D * 2;  // bytes to the tensor's end
    const int nrec = (int)(range > 0x7fffffffLL ? 0x7fffffffLL : (range > 0 ? range : 0));
    const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc((void*)(Kg + off), (short)0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc((void*)(Vg + off), (short)0, nrec, 0x00020000);
    kr = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kres, lane_off, 0, 0));
    vr = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, lane_off, 0, 0));
  };
  // V' is staged negated (rows past the end become -0, which adds nothing).
  auto store_tile = [&](int i, const u32x4& kr, const u32x4& vr) {
    const int buf = i % KV_BUFS;
    lst16(lds + OFF_K + buf * TSZ + o_stage, kr);
    lst16(lds + OFF_V + buf * TSZ + o_stage, vr ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u});
  };

  u32x4 kr0, vr0, kr1, vr1;
  if (nt > 0) {
    load_tile(0, kr0, vr0);
    store_tile(0, kr0, vr0);
    load_tile(1, kr1, vr1);
    load_tile(2, kr0, vr0);
  }

  lu16* const Yt = lds + OFF_Y;
  auto body = [&](int i, u32x4& krs, u32x4& vrs) {
    const lu16* Kc = lds + OFF_K + (i % KV_BUFS) * TSZ;
    const lu16* Vc = lds + OFF_V + (i % KV_BUFS) * TSZ;
    __syncthreads();  // B0: tile i staged; everything of tile i-1 consumed

    // G, U (tokens x this wave's hidden units): element r is token
    // 8(r/4) + 4hh + r%4, hidden unit 32w + l32.
    f32x16 accG = f32x16{}, accU = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 a = lop(Kc + o_row + 16 * ks);
      accG = mfma32(a, WgB[ks], accG);
      accU = mfma32(a, WuB[ks], accU);
    }

    // SwiGLU: s = sigmoid(G), A = G s, H = A U, gp = U silu'(G) = U s + H (1 - s).
    // A and gp stay in fp32 registers until the backward step.
    float Af[16], GPf[16];
    float Hf[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float g = accG[r];
      const float u = accU[r];
      const float s = sigmoid_fast(g);
      const float a = g * s;
      const float h = a * u;
      Af[r] = a;
      Hf[r] = h;
      GPf[r] = fmaf(-h, s, fmaf(u, s, h));
    }
    bf16x8 Hop[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      Hop[ks] = pack8(&Hf[8 * ks]);
      if (!DOT) {
        const u32x4 hv = as_u32x4(Hop[ks]);
        lu16* hp = lds + OFF_H + o_hst + 16 * ks;
        lst8(hp, u32x2{hv[0], hv[1]});
        lst8(hp + 8, u32x2{hv[2], hv[3]});
      }
    }
    // Stage tile i+1 (loaded two tiles ago) and start loading i+3 into its registers.
    if (i + 1 < nt) store_tile(i + 1, krs, vrs);
    load_tile(i + 3, krs, vrs);
    if (!DOT) __syncthreads();  // B1: H(i) complete

    // Y (tokens 16tb.., outputs 16(ob+b)..) = H W_d over all hidden units;
    // R = Y - V'; Y -> LDS [t][o].
    if (!DOT) {
      f32x4 accY[2] = {f32x4{}, f32x4{}};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const lu16* hp = lds + OFF_H + o_ha + 32 * ks * HPT;
        const bf16x8 ha = ltr_op(hp, hp + 4 * HPT);
#pragma unroll
        for (int b = 0; b < 2; ++b)
          accY[b] = mfma16(ha, lop(lds + OFF_WT + o_wtb + 16 * b * WTP + 32 * ks), accY[b]);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (LOSS) {
          const u32x2 vn = ltr(Vc + o_vl + 16 * b);
          const float r0 = accY[b][0] + bf16_lo(vn[0]);
          const float r1 = accY[b][1] + bf16_hi(vn[0]);
          const float r2 = accY[b][2] + bf16_lo(vn[1]);
          const float r3 = accY[b][3] + bf16_hi(vn[1]);
          loss = fmaf(r0, r0, loss);
          loss = fmaf(r1, r1, loss);
          loss = fmaf(r2, r2, loss);
          loss = fmaf(r3, r3, loss);
        }
        const uint32_t y01 = pack_bf16x2(accY[b][0], accY[b][1]);
        const uint32_t y23 = pack_bf16x2(accY[b][2], accY[b][3]);
        lst8(Yt + o_yst + 16 * b * YP, u32x2{y01, y23});
      }
    }
    if (!DOT) __syncthreads();  // B2: Y(i) complete

    // dH = (Y - V') W_d^T (dot loss: -V' W_d^T) for this wave's hidden units;
    // dU = dH A, dG = dH gp.
    bf16x8 dGop[2], dUop[2];
    {
      f32x16 accH = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 wdt = lop(lds + OFF_W + o_wrow + 16 * ks);  // B[k = o][j = hid]
        if (!DOT) {
          const lu16* yp = Yt + o_ytr + 16 * ks * YP;
          accH = mfma32(ltr_op(yp, yp + 4 * YP), wdt, accH);
        }
        accH = mfma32(lop(Vc + o_row + 16 * ks), wdt, accH);
      }
      if (DOT && LOSS) {
#pragma unroll
        for (int r = 0; r < 16; ++r) loss = fmaf(Hf[r], accH[r], loss);
      }
      float dg[16], du[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        du[r] = accH[r] * Af[r];
        dg[r] = accH[r] * GPf[r];
      }
      dGop[0] = pack8(&dg[0]);
      dGop[1] = pack8(&dg[8]);
      dUop[0] = pack8(&du[0]);
      dUop[1] = pack8(&du[8]);
    }

    // Weight gradients of tile i (k-slot jj of k-step ks is token
    // 16ks + 8(jj/4) + 4hh + jj%4, the register order of C tiles).
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const lu16* yt = Yt + (32 * nb + l32) * YP + 16 * ks + 4 * hh;
        const lu16* vt = Vc + o_tr + 16 * ks * TP + 32 * nb;
        if (!DOT) {
          const u32x2 y0 = *(const lu32x2*)yt, y1 = *(const lu32x2*)(yt + 8);
          accWd[nb] = mfma32(Hop[ks], as_bf16x8(u32x4{y0[0], y0[1], y1[0], y1[1]}), accWd[nb]);
        }
        accWd[nb] = mfma32(Hop[ks], ltr_op(vt, vt + 8 * TP), accWd[nb]);
      }
#pragma unroll
      for (int eb = 0; eb < 2; ++eb) {
        const lu16* kt = Kc + o_tr + 16 * ks * TP + 32 * eb;
        const bf16x8 kA = ltr_op(kt, kt + 8 * TP);
        accWg[eb] = mfma32(kA, dGop[ks], accWg[eb]);
        accWu[eb] = mfma32(kA, dUop[ks], accWu[eb]);
      }
    }
  };
  // Whole pairs in the loop (no conditional body, so the compiler's load waits
  // stay exact across iterations), an odd last tile after it.
  int i = 0;
  for (; i + 1 < nt; i += 2) {
    body(i, kr1, vr1);
    body(i + 1, kr0, vr0);
  }
  if (i < nt) body(i, kr1, vr1);

  // Partials in theta layout, times 2/d (mean squared error) or 1 (dot loss).
  constexpr float kScale = DOT ? 1.0f : 2.0f / D;
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
  if (!LOSS) {
    if (tid == 0) loss_part[(int64_t)head * P + chunk] = __builtin_nanf("");
    return;
  }
  loss = wave_sum(loss);
  if (lane == 0) red[w] = loss;
  __syncthreads();
  if (tid == 0)
    loss_part[(int64_t)head * P + chunk] = ((red[0] + red[1]) + (red[2] + red[3])) * (DOT ? 1.0f : 1.0f / D);
}

}  // namespace

hipError_t launch_grad_partial_bf16(const void* K, const void* Vp, const float* theta, float* part,
                                    float* loss_part, int64_t n_tokens, int n_heads, int P, bool dot, bool loss,
                                    hipStream_t stream) {
  const int64_t n_blocks = (int64_t)n_heads * P;
  auto kernel = dot ? (loss ? grad_partial_bf16_kernel<true, true> : grad_partial_bf16_kernel<true, false>)
                    : (loss ? grad_partial_bf16_kernel<false, true> : grad_partial_bf16_kernel<false, false>);
  hipLaunchKernelGGL(kernel, dim3((unsigned)n_blocks), dim3(256), 0, stream, static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(Vp), theta, part, loss_part, n_tokens, n_heads, P, n_blocks);
  return hipGetLastError();
}

}  // namespace vggt3

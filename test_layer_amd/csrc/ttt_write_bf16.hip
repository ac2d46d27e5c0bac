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
//
// The squared-error pass without the loss value (the write step's own case)
// runs grad_partial_mse_pipe_kernel instead: the same arithmetic, software-
// pipelined so that each wave's SwiGLU of tile c is interleaved with its
// weight-gradient MFMAs of tile c-1 (a wave overlaps its own vector and MFMA
// instructions, while vector-only and MFMA-only phases of different waves
// hardly overlap), with K, V' in three-slot rings and two barriers per tile.
//
// FUSE: the ShortConv2D in front of the write ("Non-Linear Spatial Mixing via
// ShortConv2D", same section) is computed inside this pass, so V' never has
// to exist in HBM: the kernel reads V, keeps a ring of 128 token rows of the
// head's channels in LDS, and each thread forms V' of one token and 8
// channels by the conv kernel's contract (same bits as the conv kernel).
// With VOUT it also stores that V'. The ring, the filters and a zero row take
// the place of the transposed W_d copy (the Y phase then reads W_d^T with
// transposing loads). The conv is about 250 vector instructions per thread
// and tile on top of the pass's own, which the MFMA work does not hide: at
// 1000 views the fused pass takes about 1.3 ms longer than the plain one, as
// long as the separate conv pass, so the split form remains the faster one.
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

constexpr int WTP = M + 8;             // pitch of W_d^T[o][hid]

// Fused ShortConv2D: V (not V') streams through a ring of RING_TOK token rows
// of this head's 64 channels (128 bytes each, unpadded), indexed by the token
// index modulo RING_TOK; a zero row after it stands in for out-of-grid taps;
// the head's 3x3 filters sit beside it as fp32 [tap][channel].
constexpr int RING_TOK = 128;
constexpr int OFF_RING = 0;
constexpr int OFF_ZERO = OFF_RING + RING_TOK * D;
constexpr int OFF_CW = OFF_ZERO + D;            // fp32, 2 elements each
constexpr int FUSE_BASE = OFF_CW + 2 * 9 * D;
constexpr int CONV_MAX_W = 47;  // widest grid row whose 3x3 window fits the ring (see the staging order)

// LDS map (elements of bf16). The fused form drops the transposed W_d copy
// to make room for the ring and reads W_d^T with transposing loads instead.
template <bool FUSE>
struct LdsMap {
  static constexpr int K = FUSE ? FUSE_BASE : 0;
  static constexpr int V = K + KV_BUFS * TSZ;
  static constexpr int Y = V + KV_BUFS * TSZ;
  static constexpr int H = Y + TSZ;
  static constexpr int W = H + M * HPT;
  static constexpr int WT = W + M * WP;
  static constexpr int ELEMS = FUSE ? WT : WT + D * WTP;
};
static_assert(LdsMap<false>::ELEMS * 2 <= 80 * 1024, "two workgroups per CU");
static_assert(LdsMap<true>::ELEMS * 2 <= 80 * 1024, "two workgroups per CU");
static_assert(FUSE_BASE % 8 == 0, "16-byte aligned tiles");

// LDS map of the software-pipelined squared-error kernel: K and -V' in rings
// of three slots.
struct PipeMap {
  static constexpr int KV_BUFS = 3;
  static constexpr int K = 0;
  static constexpr int V = K + KV_BUFS * TSZ;
  static constexpr int Y = V + KV_BUFS * TSZ;
  static constexpr int H = Y + TSZ;
  static constexpr int W = H + M * HPT;
  static constexpr int WT = W + M * WP;
  static constexpr int ELEMS = WT + D * WTP;
};
static_assert(PipeMap::ELEMS * 2 <= 80 * 1024, "two workgroups per CU");
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

// Workgroup barrier that the compiler's scheduler may not move any
// instruction across (by default it moves register-only work such as MFMAs
// freely past s_barrier, which would undo a hand-laid instruction mix).
__device__ __forceinline__ void segment_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

template <bool DOT, bool LOSS, bool FUSE, bool VOUT>
__global__ __launch_bounds__(256, 2) void grad_partial_bf16_kernel(
    const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg, const float* __restrict__ theta,
    float* __restrict__ part, float* __restrict__ loss_part, int64_t n_tokens, int n_heads, int P,
    int64_t n_blocks, const float* __restrict__ cw, uint16_t* __restrict__ Vpo, ConvGeom geo) {
  typedef LdsMap<FUSE> Map;
  constexpr int OFF_K = Map::K, OFF_V = Map::V, OFF_Y = Map::Y, OFF_H = Map::H, OFF_W = Map::W, OFF_WT = Map::WT;
  __shared__ __attribute__((aligned(16))) uint16_t smem[Map::ELEMS];
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
  if (!DOT && !FUSE) {
    for (int idx = tid; idx < M * D / 2; idx += 256) {
      const int o = (2 * idx) / M, hid = (2 * idx) % M;
      *(__attribute__((address_space(3))) uint32_t*)(lds + OFF_WT + o * WTP + hid) =
          pack_bf16x2(Wd[hid * D + o], Wd[(hid + 1) * D + o]);
    }
  }

  typedef __attribute__((address_space(3))) float lf32;
  typedef __attribute__((address_space(3))) f32x4 lf32x4;
  lf32* const cwl = (lf32*)(lds + OFF_CW);
  if constexpr (FUSE) {
    for (int idx = tid; idx < 9 * D; idx += 256) {
      const int tap = idx / D, ch = idx % D;
      cwl[idx] = cw[((int64_t)head * D + ch) * 9 + tap];
    }
    if (tid < 8) lst16(lds + OFF_ZERO + 8 * tid, u32x4{0u, 0u, 0u, 0u});
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
  const int o_wtr = (8 * g4 + jr) * WP + 16 * ob + 4 * q4;  // fused form: the same by transposing W_d reads
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
  auto load_k = [&](int i, u32x4& kr) {
    const int64_t t0 = (tile_begin + i) * T;
    const int64_t off = t0 * C + (int64_t)head * D;
    const int64_t range = (n_tokens - t0) * C * 2 - (int64_t)head * D * 2;
    const int nrec = (int)(range > 0x7fffffffLL ? 0x7fffffffLL : (range > 0 ? range : 0));
    const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc((void*)(Kg + off), (short)0, nrec, 0x00020000);
    kr = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kres, lane_off, 0, 0));
  };
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
    if constexpr (!FUSE)
      lst16(lds + OFF_V + buf * TSZ + o_stage, vr ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u});
  };

  // Fused form. V tile u holds tokens t_c - 48 + 32u .. + 31 (t_c: the chunk's
  // first token). Before the first tile, V tiles 0..3 are staged and V'(0) is
  // computed from them. body(i) stages V tile i + 4 right after its first
  // barrier (over rows that only V'(i), computed before that barrier, read)
  // and computes V'(i + 1) after its second barrier, at the end of the tile:
  // the ring then holds tokens [t_c + 32i - 16, t_c + 32i + 112), and the
  // window of V'(i + 1), tokens t_c + 32(i + 1) - w - 1 .. t_c + 32(i + 1) + 31
  // + w + 1 with w = grid_w <= CONV_MAX_W, lies inside it.
  const int64_t t_c = tile_begin * T;
  auto load_v = [&](int u, u32x4& vr) {
    const int64_t t0 = t_c - 48 + 32 * (int64_t)u;
    const int64_t tb = t0 < 0 ? 0 : t0;  // before token 0: rows with negative offsets read as zeros
    const int64_t off = tb * C + (int64_t)head * D;
    const int64_t range = (n_tokens - tb) * C * 2 - (int64_t)head * D * 2;
    const int nrec = (int)(range > 0x7fffffffLL ? 0x7fffffffLL : (range > 0 ? range : 0));
    const int voff = lane_off + (t0 < 0 ? (int)(t0 * C * 2) : 0);
    const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc((void*)(Vg + off), (short)0, nrec, 0x00020000);
    vr = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, voff, 0, 0));
  };
  auto stage_v = [&](int u, const u32x4& vr) {
    const int r0 = (int)((t_c - 48 + 32 * (int64_t)u) & (RING_TOK - 1));
    lst16(lds + OFF_RING + ((r0 + srow) & (RING_TOK - 1)) * D + scol, vr);
  };
  // V'(j) of this lane's token and 8 channels by the conv contract: acc = +0,
  // taps row offset outermost, column offset innermost, acc = fl(acc + fl(w v))
  // with no fused multiply-add; out-of-grid taps read the zero row (adding
  // fl(w * 0) = +-0 leaves acc unchanged, as skipping them would); special
  // tokens pass V through; rows at or past n_tokens stage zeros.
  auto conv_tile = [&](int j, uint32_t cpos) {
    const int64_t t0 = (tile_begin + j) * T;
    const int64_t left = n_tokens - t0;
    const bool valid = srow < (left > T ? T : (int)left);
    const uint32_t p = cpos + (uint32_t)srow;
    const uint32_t q = geo.magic_tpv ? __umulhi(p, geo.magic_tpv) : p;
    const int pos = (int)(p - q * (uint32_t)geo.tpv);
    const bool special = pos < geo.n_special;
    const uint32_t pp = (uint32_t)(pos - geo.n_special);
    const uint32_t yy = geo.magic_gw ? __umulhi(pp, geo.magic_gw) : pp;
    const int y = (int)yy, x = (int)(pp - yy * (uint32_t)geo.grid_w);
    const bool up = y > 0, dn = y < geo.grid_h - 1, lf = x > 0, rt = x < geo.grid_w - 1;
    const uint32_t c7 = (uint32_t)((int)(t0 & (RING_TOK - 1)) + srow) << 7;
    const uint32_t oc16 = (uint32_t)scol * 2;
    const uint32_t zaddr = (uint32_t)(RING_TOK * 128) + oc16;
    const __attribute__((address_space(3))) uint8_t* ring = (const __attribute__((address_space(3))) uint8_t*)(lds + OFF_RING);
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    u32x4 center = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int dy = 0; dy < 3; ++dy) {
#pragma unroll
      for (int dx = 0; dx < 3; ++dx) {
        const int off = (dy - 1) * geo.grid_w + (dx - 1);
        uint32_t a = ((c7 + (uint32_t)(off * 128)) & (uint32_t)((RING_TOK - 1) << 7)) | oc16;
        bool ok = true;
        if (dy == 0) ok = up;
        if (dy == 2) ok = dn;
        if (dx == 0) ok = ok && lf;
        if (dx == 2) ok = ok && rt;
        if (dy != 1 || dx != 1) a = ok ? a : zaddr;
        const u32x4 v = *(const lu32x4*)(ring + a);
        if (dy == 1 && dx == 1) center = v;
        const int tap = 3 * dy + dx;
        const f32x4 w0 = *(const lf32x4*)(cwl + tap * D + scol);
        const f32x4 w1 = *(const lf32x4*)(cwl + tap * D + scol + 4);
        {
#pragma clang fp contract(off)
          acc[0] = acc[0] + w0[0] * bf16_lo(v[0]);
          acc[1] = acc[1] + w0[1] * bf16_hi(v[0]);
          acc[2] = acc[2] + w0[2] * bf16_lo(v[1]);
          acc[3] = acc[3] + w0[3] * bf16_hi(v[1]);
          acc[4] = acc[4] + w1[0] * bf16_lo(v[2]);
          acc[5] = acc[5] + w1[1] * bf16_hi(v[2]);
          acc[6] = acc[6] + w1[2] * bf16_lo(v[3]);
          acc[7] = acc[7] + w1[3] * bf16_hi(v[3]);
        }
      }
    }
    u32x4 res = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                 pack_bf16x2(acc[6], acc[7])};
    if (special) res = center;
    if (!valid) res = u32x4{0u, 0u, 0u, 0u};
    lst16(lds + OFF_V + (j % KV_BUFS) * TSZ + o_stage, res ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u});
    if constexpr (VOUT) {
      const int64_t off = t0 * C + (int64_t)head * D;
      const int64_t range = left * C * 2 - (int64_t)head * D * 2;
      const int nrec = (int)(range > 0x7fffffffLL ? 0x7fffffffLL : (range > 0 ? range : 0));
      const __amdgpu_buffer_rsrc_t ores = __builtin_amdgcn_make_buffer_rsrc((void*)(Vpo + off), (short)0, nrec, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b128(res, ores, lane_off, 0, 0);
    }
  };
  uint32_t cpos = 0;  // position within its view of the first token of the tile being convolved
  if constexpr (FUSE) cpos = (uint32_t)(t_c % geo.tpv);

  u32x4 kr0, vr0, kr1, vr1;
  if constexpr (!FUSE) {
    if (nt > 0) {
      load_tile(0, kr0, vr0);
      store_tile(0, kr0, vr0);
      load_tile(1, kr1, vr1);
      load_tile(2, kr0, vr0);
    }
  } else if (nt > 0) {
    load_k(0, kr0);
    store_tile(0, kr0, vr0);
    u32x4 va, vb, vc, vd;
    load_v(0, va);
    load_v(1, vb);
    load_v(2, vc);
    load_v(3, vd);
    stage_v(0, va);
    stage_v(1, vb);
    stage_v(2, vc);
    stage_v(3, vd);
    __syncthreads();  // V tiles 0..3 and the filters staged
    conv_tile(0, cpos);
    load_k(1, kr1);
    load_v(4, vr1);
    load_k(2, kr0);
    load_v(5, vr0);
  }

  lu16* const Yt = lds + OFF_Y;
  auto body = [&](int i, u32x4& krs, u32x4& vrs) {
    const lu16* Kc = lds + OFF_K + (i % KV_BUFS) * TSZ;
    const lu16* Vc = lds + OFF_V + (i % KV_BUFS) * TSZ;
    __syncthreads();  // B0: tile i staged; everything of tile i-1 consumed
    if constexpr (FUSE) {
      stage_v(i + 4, vrs);  // over rows the window of V'(i) (computed before B0) was the last to read
      load_v(i + 6, vrs);
    }

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
    if constexpr (FUSE) load_k(i + 3, krs);
    else load_tile(i + 3, krs, vrs);
    if (!DOT || FUSE) __syncthreads();  // B1: H(i) complete; the conv window of V'(i+1) read

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
          if constexpr (FUSE) {
            const lu16* wp = lds + OFF_W + o_wtr + 32 * ks * WP + 16 * b;
            accY[b] = mfma16(ha, ltr_op(wp, wp + 4 * WP), accY[b]);
          } else {
            accY[b] = mfma16(ha, lop(lds + OFF_WT + o_wtb + 16 * b * WTP + 32 * ks), accY[b]);
          }
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
    // V'(i + 1) into the slot tile i-1 released, from the ring as staged
    // before B1.
    if constexpr (FUSE) {
      if (i + 1 < nt) {
        cpos += T;
        while (cpos >= (uint32_t)geo.tpv) cpos -= (uint32_t)geo.tpv;
        conv_tile(i + 1, cpos);
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

// The squared-error gradient without the loss value (what a write step with
// no loss output needs), software-pipelined across tiles. Same partials, bit
// for bit, as grad_partial_bf16_kernel<false, false, false, false>: every
// accumulator receives the same MFMA terms in the same order.
__global__ __launch_bounds__(256, 2) void grad_partial_mse_pipe_kernel(
    const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg, const float* __restrict__ theta,
    float* __restrict__ part, float* __restrict__ loss_part, int64_t n_tokens, int n_heads, int P,
    int64_t n_blocks) {
  constexpr int KV_BUFS = PipeMap::KV_BUFS;
  constexpr int OFF_K = PipeMap::K, OFF_V = PipeMap::V, OFF_Y = PipeMap::Y, OFF_H = PipeMap::H, OFF_W = PipeMap::W,
                OFF_WT = PipeMap::WT;
  __shared__ __attribute__((aligned(16))) uint16_t smem[PipeMap::ELEMS];
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
  for (int idx = tid; idx < M * D / 2; idx += 256) {
    const int o = (2 * idx) / M, hid = (2 * idx) % M;
    *(__attribute__((address_space(3))) uint32_t*)(lds + OFF_WT + o * WTP + hid) =
        pack_bf16x2(Wd[hid * D + o], Wd[(hid + 1) * D + o]);
  }

  f32x16 accWd[2], accWg[2], accWu[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    accWd[i] = f32x16{};
    accWg[i] = f32x16{};
    accWu[i] = f32x16{};
  }
  const int64_t n_tiles_all = (n_tokens + T - 1) / T;
  const int64_t tile_begin = n_tiles_all * chunk / P;
  const int nt = (int)(n_tiles_all * (chunk + 1) / P - tile_begin);

  // Lane-constant LDS offsets (elements).
  const int o_row = l32 * TP + 8 * hh;                     // token-row operand reads (b128)
  const int o_tr = (4 * hh + jr) * TP + cb + 4 * q4;        // transpose reads over token rows
  const int o_hst = (32 * w + l32) * HPT + 4 * hh;          // H stores
  const int o_ha = (8 * g4 + jr) * HPT + 16 * tb + 4 * q4;  // Y phase: H^T reads (A operand)
  const int o_wtb = (16 * ob + i16) * WTP + 8 * g4;         // Y phase: W_d^T reads (B operand)
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
  auto store_tile = [&](int buf, const u32x4& kr, const u32x4& vr) {
    lst16(lds + OFF_K + buf * TSZ + o_stage, kr);
    lst16(lds + OFF_V + buf * TSZ + o_stage, vr ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u});
  };

  u32x4 kr0, vr0, kr1, vr1;
  lu16* const Yt = lds + OFF_Y;

  // Carried from one tile to the next: the previous tile's weight-gradient operands.
  bf16x8 HopP[2], dGopP[2], dUopP[2];

  // G, U (tokens x this wave's hidden units) of tile i from K(i) in LDS:
  // element r is token 8(r/4) + 4hh + r%4, hidden unit 32w + l32.
  auto gate_up = [&](int sl, f32x16& accG, f32x16& accU) {
    const lu16* Kc = lds + OFF_K + sl * TSZ;
    accG = f32x16{};
    accU = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 a = lop(Kc + o_row + 16 * ks);
      accG = mfma32(a, WgB[ks], accG);
      accU = mfma32(a, WuB[ks], accU);
    }
  };

  // Weight gradients of tile i from its carried operands (k-slot jj of k-step
  // ks is token 16ks + 8(jj/4) + 4hh + jj%4, the register order of C tiles),
  // as a fixed sequence of 8 MFMA steps per k-step ks: gW_d block 0 against Y
  // then -V', block 1 likewise, then gW_g, gW_u against K block 0, then block
  // 1. Each accumulator sees its terms in the same order as in
  // grad_partial_bf16_kernel, so the partials are bitwise the same.
  constexpr int WG_STEPS = 16;
  constexpr int PER_KS = WG_STEPS / 2;
  // LDS operand of step k (the B operand of a gW_d step, the K operand of a
  // gW_g step; a gW_u step reuses the K operand of the step before it).
  auto wg_reuses = [](int k) { const int j = k % PER_KS; return j >= PER_KS - 4 && (j - (PER_KS - 4)) % 2 == 1; };
  auto wg_operand = [&](int sl, int k) -> bf16x8 {
    const lu16* Kc = lds + OFF_K + sl * TSZ;
    const lu16* Vc = lds + OFF_V + sl * TSZ;
    const int ks = k / PER_KS, j = k % PER_KS;
    if (j < PER_KS - 4) {  // gW_d step
      const int nb = j / 2;
      if (j % 2 == 0) {
        const lu16* yt = Yt + (32 * nb + l32) * YP + 16 * ks + 4 * hh;
        const u32x2 y0 = *(const lu32x2*)yt, y1 = *(const lu32x2*)(yt + 8);
        return as_bf16x8(u32x4{y0[0], y0[1], y1[0], y1[1]});
      }
      const lu16* vt = Vc + o_tr + 16 * ks * TP + 32 * nb;
      return ltr_op(vt, vt + 8 * TP);
    }
    const int eb = (j - (PER_KS - 4)) / 2;
    const lu16* kt = Kc + o_tr + 16 * ks * TP + 32 * eb;
    return ltr_op(kt, kt + 8 * TP);
  };
  auto wg_mfma = [&](int k, const bf16x8& op) {
    const int ks = k / PER_KS, j = k % PER_KS;
    if (j < PER_KS - 4) {
      const int nb = j / 2;
      accWd[nb] = mfma32(HopP[ks], op, accWd[nb]);
    } else {
      const int e = j - (PER_KS - 4), eb = e / 2;
      if (e % 2 == 0) accWg[eb] = mfma32(op, dGopP[ks], accWg[eb]);
      else accWu[eb] = mfma32(op, dUopP[ks], accWu[eb]);
    }
  };
  auto weight_grads = [&](int i) {
#pragma unroll
    for (int k = 0; k < WG_STEPS; ++k) {
      const bf16x8 op = wg_operand(i % KV_BUFS, wg_reuses(k) ? k - 1 : k);
      wg_mfma(k, op);
    }
  };

  // One tile, software-pipelined so that each wave's instruction stream mixes
  // matrix and vector work: the SwiGLU of tile i (vector ALU) is interleaved
  // with the weight-gradient MFMAs of tile i-1, which do not depend on it.
  //   A | G, U(i) ; SwiGLU(i) -> H(i) with weight grads(i-1) ; stage K,V'(i+1), load i+3
  //   B1| Y(i) = H(i) W_d (16x16x32 tiles over all hidden units) ; Y -> LDS [o][t]
  //   B2| dH(i) = (Y - V') W_d^T ; dG, dU
  // K and V' tiles live in a ring of three LDS slots: tile i-1 is read in A
  // while tile i+1 is written there, tile i stays for B1/B2.
  // On one SIMD, vector instructions overlap an MFMA of the same wave almost
  // for free, while a wave of only vector work beside a wave of only MFMAs
  // slows both down. Segment A is therefore laid out by hand: the SwiGLU runs
  // in four groups of four elements (stage by stage within a group, so that
  // consecutive instructions are independent), cut into one chunk per MFMA;
  // each MFMA's LDS operand is read two MFMAs ahead; sched_barrier fences keep
  // the compiler from regrouping the chunks.
  // sl = i % KV_BUFS, passed as a literal so that every slot offset folds
  // into the LDS instructions' immediate offsets.
  auto body = [&](int i, int sl, u32x4& krs, u32x4& vrs, bool first) __attribute__((always_inline)) {
    const int slp = (sl + KV_BUFS - 1) % KV_BUFS, sln = (sl + 1) % KV_BUFS;
    const lu16* Vc = lds + OFF_V + sl * TSZ;
    f32x16 accG, accU;
    gate_up(sl, accG, accU);
    bf16x8 opr[WG_STEPS];
    if (!first) {
      opr[0] = wg_operand(slp, 0);
      opr[1] = wg_operand(slp, 1);
    }
    __builtin_amdgcn_sched_barrier(0);

    // SwiGLU: s = sigmoid(G), A = G s, H = A U, gp = U silu'(G) = U s + H (1 - s),
    // with sigmoid(g) = 1 / (1 + 2^(-g log2 e)). A and gp stay in fp32
    // registers until the backward step.
    float Af[16], GPf[16], Hf[16], X[16];
    uint32_t Hpk[8];
    constexpr int OPS = 34;  // per group of four elements: 8 stages x 4, then 2 packs
    auto sw_op = [&](int grp, int o) {
      if (o >= 32) {
        const int r = 4 * grp + 2 * (o - 32);
        Hpk[r / 2] = pack_bf16x2(Hf[r], Hf[r + 1]);
        return;
      }
      const int r = 4 * grp + o % 4;
      const float g = accG[r], u = accU[r];
      switch (o / 4) {
        case 0: X[r] = g * -1.4426950408889634f; break;
        case 1: X[r] = __builtin_amdgcn_exp2f(X[r]); break;
        case 2: X[r] = 1.0f + X[r]; break;
        case 3: X[r] = __builtin_amdgcn_rcpf(X[r]); break;
        case 4: Af[r] = g * X[r]; break;
        case 5: Hf[r] = Af[r] * u; break;
        case 6: GPf[r] = fmaf(u, X[r], Hf[r]); break;
        default: GPf[r] = fmaf(-Hf[r], X[r], GPf[r]); break;
      }
    };
    constexpr int MPG = WG_STEPS / 4;  // MFMAs per group
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
#pragma unroll
      for (int c = 0; c < MPG; ++c) {
        const int k = grp * MPG + c;
        if (!first) {
          if (k + 2 < WG_STEPS && !wg_reuses(k + 2)) opr[k + 2] = wg_operand(slp, k + 2);
          wg_mfma(k, opr[wg_reuses(k) ? k - 1 : k]);
        }
#pragma unroll
        for (int o = c * OPS / MPG; o < (c + 1) * OPS / MPG; ++o) sw_op(grp, o);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    bf16x8 Hop[2];
    Hop[0] = as_bf16x8(u32x4{Hpk[0], Hpk[1], Hpk[2], Hpk[3]});
    Hop[1] = as_bf16x8(u32x4{Hpk[4], Hpk[5], Hpk[6], Hpk[7]});
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      lu16* hp = lds + OFF_H + o_hst + 16 * ks;
      lst8(hp, u32x2{Hpk[4 * ks], Hpk[4 * ks + 1]});
      lst8(hp + 8, u32x2{Hpk[4 * ks + 2], Hpk[4 * ks + 3]});
    }
    // Stage tile i+1 (loaded two tiles ago) and start loading i+3 into its registers.
    if (i + 1 < nt) store_tile(sln, krs, vrs);
    load_tile(i + 3, krs, vrs);
    segment_barrier();  // B1: H(i) and K,V'(i+1) staged; tile i-1 and Y(i-1) consumed

    // Y (tokens 16tb.., outputs 16(ob+b)..) = H W_d over all hidden units;
    // Y -> LDS [o][t].
    {
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
        const uint32_t y01 = pack_bf16x2(accY[b][0], accY[b][1]);
        const uint32_t y23 = pack_bf16x2(accY[b][2], accY[b][3]);
        lst8(Yt + o_yst + 16 * b * YP, u32x2{y01, y23});
      }
      segment_barrier();  // B2: Y(i) complete
    }

    // dH = (Y - V') W_d^T for this wave's hidden units; dU = dH A, dG = dH gp.
    {
      f32x16 accH = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 wdt = lop(lds + OFF_W + o_wrow + 16 * ks);  // B[k = o][j = hid]
        const lu16* yp = Yt + o_ytr + 16 * ks * YP;
        accH = mfma32(ltr_op(yp, yp + 4 * YP), wdt, accH);
        accH = mfma32(lop(Vc + o_row + 16 * ks), wdt, accH);
      }
      float dg[16], du[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        du[r] = accH[r] * Af[r];
        dg[r] = accH[r] * GPf[r];
      }
      dGopP[0] = pack8(&dg[0]);
      dGopP[1] = pack8(&dg[8]);
      dUopP[0] = pack8(&du[0]);
      dUopP[1] = pack8(&du[8]);
      HopP[0] = Hop[0];
      HopP[1] = Hop[1];
    }
  };

  if (nt > 0) {
    load_tile(0, kr0, vr0);
    store_tile(0, kr0, vr0);
    load_tile(1, kr1, vr1);
    load_tile(2, kr0, vr0);
    segment_barrier();  // K, V'(0) staged
    body(0, 0, kr1, vr1, true);
  }
  // Six tiles per iteration (two register sets x three LDS slots, so every
  // slot offset is a constant), no conditional body inside the loop; the
  // remaining tiles after it.
  int i = 1;
  for (; i + 5 < nt; i += 6) {
    body(i, 1, kr0, vr0, false);
    body(i + 1, 2, kr1, vr1, false);
    body(i + 2, 0, kr0, vr0, false);
    body(i + 3, 1, kr1, vr1, false);
    body(i + 4, 2, kr0, vr0, false);
    body(i + 5, 0, kr1, vr1, false);
  }
  if (i < nt) body(i, 1, kr0, vr0, false);
  if (i + 1 < nt) body(i + 1, 2, kr1, vr1, false);
  if (i + 2 < nt) body(i + 2, 0, kr0, vr0, false);
  if (i + 3 < nt) body(i + 3, 1, kr1, vr1, false);
  if (i + 4 < nt) body(i + 4, 2, kr0, vr0, false);
  if (nt > 0) weight_grads(nt - 1);

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
  if (tid == 0) loss_part[(int64_t)head * P + chunk] = __builtin_nanf("");
}


}  // namespace

hipError_t launch_grad_partial_bf16(const void* K, const void* Vp, const float* theta, float* part,
                                    float* loss_part, int64_t n_tokens, int n_heads, int P, bool dot, bool loss,
                                    hipStream_t stream) {
  const int64_t n_blocks = (int64_t)n_heads * P;
  const uint16_t* Kb = static_cast<const uint16_t*>(K);
  const uint16_t* Vb = static_cast<const uint16_t*>(Vp);
  if (!dot && !loss) {
    hipLaunchKernelGGL(grad_partial_mse_pipe_kernel, dim3((unsigned)n_blocks), dim3(256), 0, stream, Kb, Vb, theta,
                       part, loss_part, n_tokens, n_heads, P, n_blocks);
    return hipGetLastError();
  }
  auto kernel = dot ? (loss ? grad_partial_bf16_kernel<true, true, false, false>
                            : grad_partial_bf16_kernel<true, false, false, false>)
                    : grad_partial_bf16_kernel<false, true, false, false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)n_blocks), dim3(256), 0, stream, Kb, Vb, theta, part, loss_part, n_tokens,
                     n_heads, P, n_blocks, nullptr, nullptr, ConvGeom{});
  return hipGetLastError();
}

int conv_fused_max_grid_w() { return CONV_MAX_W; }

hipError_t launch_grad_partial_conv_bf16(const void* K, const void* V, const float* conv_w, void* Vp_out,
                                         const ConvGeom& geo, const float* theta, float* part, float* loss_part,
                                         int64_t n_tokens, int n_heads, int P, bool dot, bool loss,
                                         hipStream_t stream) {
  const int64_t n_blocks = (int64_t)n_heads * P;
  typedef void (*kfn)(const uint16_t*, const uint16_t*, const float*, float*, float*, int64_t, int, int, int64_t,
                      const float*, uint16_t*, ConvGeom);
  kfn kernel;
  if (Vp_out)
    kernel = dot ? (loss ? grad_partial_bf16_kernel<true, true, true, true> : grad_partial_bf16_kernel<true, false, true, true>)
                 : (loss ? grad_partial_bf16_kernel<false, true, true, true> : grad_partial_bf16_kernel<false, false, true, true>);
  else
    kernel = dot ? (loss ? grad_partial_bf16_kernel<true, true, true, false> : grad_partial_bf16_kernel<true, false, true, false>)
                 : (loss ? grad_partial_bf16_kernel<false, true, true, false> : grad_partial_bf16_kernel<false, false, true, false>);
  hipLaunchKernelGGL(kernel, dim3((unsigned)n_blocks), dim3(256), 0, stream, static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), theta, part, loss_part, n_tokens, n_heads, P, n_blocks, conv_w,
                     static_cast<uint16_t*>(Vp_out), geo);
  return hipGetLastError();
}

}  // namespace vggt3


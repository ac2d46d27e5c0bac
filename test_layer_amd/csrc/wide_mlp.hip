// Wide fast-weight MLP: one SwiGLU T(x) = (silu(x W_g) * (x W_u)) W_d over the
// whole token width, d = 1024 inputs/outputs and m = 4096 hidden units
// (paper-graph summary "VGG-T3: Offline Feed-Forward 3D Reconstruction at
// Scale", section 3.4 "TTT MLP Architecture and Inner Optimization": a
// 1024 -> 4096 -> 1024 SwiGLU; biases are left out as in the per-head layer).
//
// At this width every phase of the write and the read is a large dense
// contraction, so the path is a sequence of bf16 MFMA GEMMs with the
// elementwise work fused into their epilogues. Per token chunk (Eq. 5 of
// "Large-Scale Inference Strategies": the gradient is a sum over minibatches):
//   P1  [G | U] = K [W_g | W_u]          epilogue: s = sigmoid(G), A = G s,
//                                        H = A U, GP = U silu'(G)
//   P2  Y = H W_d                        epilogue: loss += (Y - V')^2, store -Y
//   P3  D = [-Y | V'] [W_d ; W_d]^T      epilogue: dG = D GP, dU = D A
//   P4  [gW_g | gW_u] += K^T [dG | dU],  gW_d += H^T (-Y) + H^T V'
// so D = -(Y - V') W_d^T and all three accumulated gradients are the true
// ones times -(d/2) (mean squared error) or -1 (dot-product loss, where
// P2 is skipped and P3 is D = V' W_d^T). The dot-product loss needs no
// per-token work: -sum_i Y_i . V'_i = <W_d, -H^T V'> = <W_d, gW_d>, a dot
// product of the weights with the reduced gradient (taken in the reduce). The residual is never rounded as a
// whole: Y (small next to V' at the start of fitting) and V' enter as two
// exact bf16 operands, as in the per-head write.
//
// GEMM tile: 256 x 256 per workgroup of 8 waves (2 x 4), 128 x 64 per wave as
// 8 x 4 tiles of v_mfma_f32_16x16x32_bf16, k blocks of 64 brought into a
// double-buffered LDS (128 KB, one workgroup per CU, two waves per SIMD) by
// direct global-to-LDS loads that overlap the previous block's MFMAs. An
// operand whose k index is contiguous in memory is kept [rows][k] in LDS and
// read with ds_read_b128; one whose rows are contiguous (the token-reduction
// GEMMs of P4) is kept [k][rows] and read with ds_read_b64_tr_b16.
#include "bf16_ops.hpp"
#include "kernels.hpp"
#include "wide.hpp"

namespace vggt3 {
namespace wide {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NTHR = 512;
constexpr int NWAVE = NTHR / 64;
constexpr int WM = 128, WN = 64;      // wave tile (2 x 4 waves)
constexpr int TM = WM / 16, TN = WN / 16;
constexpr int TSZ = 256 * BK;         // elements of one operand tile (32 KB)

typedef __attribute__((address_space(3))) uint16_t lu16;
typedef __attribute__((address_space(3))) u32x4 lu32x4;
typedef __attribute__((address_space(3))) u32x2 lu32x2;
typedef __attribute__((address_space(3))) void lvoid;

__device__ __forceinline__ bf16x8 lop(const lu16* p) {
  const u32x4 v = *(const lu32x4*)p;
  return as_bf16x8(v);
}
__device__ __forceinline__ u32x2 ltr(const lu16* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}
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

// LDS tiles, 16-byte pieces, unpadded and XOR-swizzled so that the operand
// reads below hit distinct banks.
//  KC tile (k contiguous in memory): [256 rows][BK]; piece (row, c) of the
//     8 per row is stored at position c ^ ((row / 2) % 8).
//  RC tile (rows contiguous in memory): [BK][256]; piece (k, c) of the 32 per
//     k row is stored at position c ^ rc_swz(k).
__device__ __forceinline__ int kc_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int rc_swz(int k) { return 2 * (k & 3) + 8 * ((k >> 3) & 1); }

// Fill one operand tile with direct global -> LDS loads (gfx950
// global_load_lds_dwordx4: lane l of a wave writes the 16 bytes at LDS base +
// 16 l). Instruction i of wave w fills pieces [(8i + w) 64, +64) of the tile;
// each lane picks the global piece that the swizzle assigns to its position.
// The address is a block-uniform base plus a 32-bit lane offset (in elements).
// KC: element (r, k) at src[r * ld + k]; rows past r_end read row r_end - 1.
// RC: element (r, k) at src[k * ld + r]; k rows past k_rows (the rows the
//     operand has) read row k_rows - 1. The K tail of a block (rows K .. the
//     next multiple of 64) thus reads, for each product, zeros from one operand
//     (a workspace buffer written with zero rows there, k_rows >= K rounded up)
//     and clamped copies from the other (k_rows = K).
template <bool KC>
__device__ __forceinline__ void dma_tile(lu16* tile, const uint16_t* src, int64_t ld, int64_t r0, int64_t r_end,
                                         int64_t k0, int64_t k_end, int wid, int lane) {
  const uint16_t* base = KC ? src + r0 * ld + k0 : src + k0 * ld + r0;
  const int rmax = KC ? (int)(r_end - r0 - 1) : (int)(k_end - k0 - 1);
#pragma unroll
  for (int i = 0; i < 2048 / NTHR; ++i) {
    const int p = (NWAVE * i + wid) * 64 + lane;
    uint32_t off;
    if (KC) {
      const int row = p >> 3;
      const int c = (p & 7) ^ kc_swz(row);
      off = (uint32_t)(row < rmax ? row : rmax) * (uint32_t)ld + 8u * c;
    } else {
      const int kr = p >> 5;
      const int c = (p & 31) ^ rc_swz(kr);
      off = (uint32_t)(kr < rmax ? kr : rmax) * (uint32_t)ld + 8u * c;
    }
    __builtin_amdgcn_global_load_lds(base + off, (lvoid*)(tile + (NWAVE * i + wid) * 512), 16, 0, 0);
  }
}

// Lane-dependent LDS offsets (elements) of the operand reads. Tile row/column
// bases are multiples of 16, so the KC swizzle of row base + i16 depends on the
// lane only and fragment i of a wave sits at a constant distance from it; the
// RC swizzle moves each 16-column group by a lane-dependent amount, so each of
// the wave's 8 fragments has its own offset (k sub-step and stage are constant
// distances from it).
struct FetchOffsets {
  int kc[2];  // KC: per k sub-step, add (row base) * BK
  int rc[8];  // RC: per fragment of the wave, add kk * 32 * 256
};
__device__ __forceinline__ FetchOffsets fetch_offsets(int wbase, int i16, int g4, int jr, int q4) {
  FetchOffsets o;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) o.kc[kk] = i16 * BK + 8 * ((kk * 4 + g4) ^ kc_swz(i16));
  const int kr = 8 * g4 + jr;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int col = wbase + 16 * i + 4 * q4;
    o.rc[i] = kr * 256 + 8 * ((col >> 3) ^ rc_swz(kr)) + 4 * ((col >> 2) & 1);
  }
  return o;
}

template <bool KC>
__device__ __forceinline__ bf16x8 fetch(const lu16* s, const FetchOffsets& o, int wbase, int i, int kk) {
  if (KC) return lop(s + (wbase + 16 * i) * BK + o.kc[kk]);
  const lu16* p = s + kk * 32 * 256 + o.rc[i];
  return ltr_op(p, p + 4 * 256);
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// C-native layout of a [R x N] matrix (R, N multiples of 16): 16x16 blocks in
// row-major block order, 256 elements each, element (lane l, register r) of
// the MFMA C tile at l * 4 + r.
__device__ __forceinline__ int64_t cn_off(int64_t row0, int64_t col0, int64_t N, int lane) {
  return ((row0 >> 4) * (N >> 4) + (col0 >> 4)) * 256 + lane * 4;
}

// Epilogue staging through LDS, one 18 KB region per wave (the GEMM tiles are
// no longer needed then). An output sub-tile of 128 rows x (8 ncc) columns is
// written transposed, [column][row] with a row pitch of EP_P elements, with
// one 8-byte write per 4 consecutive rows of a column (the MFMA C layout), and
// read back with the transpose read so that each lane holds 8 consecutive
// columns of one row: 16-byte global stores instead of 2-byte ones.
constexpr int EP_P = 144;
constexpr int EP_ELEMS = 64 * EP_P;  // per wave
constexpr int VP_P = 72;             // pitch of a wave's row-major [128][64] input tile
static_assert(128 * VP_P <= EP_ELEMS, "input staging");
constexpr int SMEM_ELEMS = NWAVE * EP_ELEMS > 4 * TSZ ? NWAVE * EP_ELEMS : 4 * TSZ;

__device__ __forceinline__ void ep_put(lu16* T, int i, int j, int i16, int g4, float v0, float v1, float v2,
                                       float v3) {
  *(lu32x2*)(T + (16 * j + i16) * EP_P + 16 * i + 4 * g4) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
}

// Rows row0 + 0..127 (those below r_end) of columns col0 + 0 .. 8*NCC-1 from
// the staged tile T to dst (row-major, leading dimension ld).
template <int NCC>
__device__ __forceinline__ void ep_flush(const lu16* T, uint16_t* dst, int64_t ld, int64_t row0, int64_t col0,
                                         int64_t r_end, int lane) {
  const int s = lane & 15, gq = lane >> 4, j = s >> 2, q = s & 3;
#pragma unroll
  for (int p = 0; p < 8 * NCC / 4; ++p) {
    const int c0 = NCC == 8 ? 16 * (p >> 1) : 16 * p;
    const int cc = NCC == 8 ? 4 * (p & 1) + gq : gq;
    const lu16* a = T + (8 * cc + j) * EP_P + c0 + 4 * q;
    const u32x2 lo = ltr(a), hi = ltr(a + 4 * EP_P);
    const int64_t row = row0 + c0 + s;
    if (row < r_end) st16(dst + row * ld + col0 + 8 * cc, u32x4{lo[0], lo[1], hi[0], hi[1]});
  }
}

__device__ __forceinline__ float block_sum(float v, float* red, int tid) {
  v = wave_sum(v);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  float s = 0.0f;
  if (tid == 0) {
    s = ((red[0] + red[1]) + (red[2] + red[3])) + ((red[4] + red[5]) + (red[6] + red[7]));
  }
  return s;
}

// One k block (two k sub-steps of 32). The A fragment of row tile i is
// reloaded for the second sub-step as soon as its first-sub-step MFMAs have
// been issued, so those loads overlap the remaining MFMAs and only 16
// fragments are live at a time.
template <bool AKC, bool BKC>
__device__ __forceinline__ void mma_stage(const lu16* As, const lu16* Bs, f32x4 (&acc)[TM][TN], int lane, int abase,
                                          int bbase) {
  // The lane's read offsets are derived here from an opaque copy of the lane
  // index, once per k block: a handful of VALU operations that keep the
  // compiler from holding every fragment's offset in a register across the loop.
  int l = lane;
  asm volatile("" : "+v"(l));
  const int i16 = l & 15, g4 = l >> 4, jr = (l & 15) >> 2, q4 = l & 3;
  const FetchOffsets oa = fetch_offsets(abase, i16, g4, jr, q4);
  const FetchOffsets ob = fetch_offsets(bbase, i16, g4, jr, q4);
  bf16x8 a[TM], b0[TN], b1[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) b0[j] = fetch<BKC>(Bs, ob, bbase, j, 0);
#pragma unroll
  for (int i = 0; i < TM; ++i) a[i] = fetch<AKC>(As, oa, abase, i, 0);
#pragma unroll
  for (int j = 0; j < TN; ++j) b1[j] = fetch<BKC>(Bs, ob, bbase, j, 1);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(a[i], b0[j], acc[i][j]);
    a[i] = fetch<AKC>(As, oa, abase, i, 1);
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(a[i], b1[j], acc[i][j]);
}

template <bool AKC, bool BKC, int EPI>
__global__ __launch_bounds__(NTHR, 1) void gemm_kernel(GemmArgs g) {
  // Two stages of (A, B) tiles: A of stage s at s * TSZ, B at (2 + s) * TSZ,
  // so that a stage's tiles are 64 KB apart and the other stage's 32 KB.
  __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM_ELEMS];
  lu16* const A0 = (lu16*)smem;
  lu16* const A1 = A0 + TSZ;
  lu16* const B0 = A0 + 2 * TSZ;
  lu16* const B1 = A0 + 3 * TSZ;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 2, wn = wid & 3;
  const int abase = wm * WM, bbase = wn * WN;

  const int64_t tiles_n = g.N / BN;
  const int64_t tiles_m = (g.M + BM - 1) / BM;
  const int64_t tiles = tiles_m * tiles_n;
  const int64_t b = xcd_remap(blockIdx.x, (int64_t)gridDim.x);
  const int slice = (int)(b / tiles);
  const int64_t t = b % tiles;
  // Tiles in groups of 4 row tiles x all column tiles, row-fastest within a
  // group: the workgroups that run together on one XCD (xcd_remap gives each
  // XCD a contiguous range) share 4 A row panels and a few B column panels in
  // its L2 instead of streaming every B panel.
  int64_t tm_, tn_;
  {
    constexpr int64_t GM = 4;
    const int64_t group = t / (GM * tiles_n), first = group * GM;
    const int64_t gsz = tiles_m - first < GM ? tiles_m - first : GM;
    const int64_t in = t % (GM * tiles_n);
    tm_ = first + in % gsz;
    tn_ = in / gsz;
  }
  const int64_t m0 = tm_ * BM, n0 = tn_ * BN;

  const int64_t nkb = (g.K + BK - 1) / BK;
  const int64_t kb0 = nkb * slice / g.S, kb1 = nkb * (slice + 1) / g.S;
  const int64_t nkr = kb1 - kb0;
  const int64_t nit = nkr * g.nseg;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Iteration it covers k block kb0 + (it mod nkr) of segment it / nkr (nseg <= 2).
  auto issue = [&](int64_t it, lu16* ta, lu16* tb) {
    const int seg = it >= nkr ? 1 : 0;
    const int64_t k0 = (kb0 + it - seg * nkr) * BK;
    dma_tile<AKC>(ta, g.A[seg], g.lda[seg], m0, g.M, k0, g.a_rows[seg], wid, lane);
    dma_tile<BKC>(tb, g.B[seg], g.ldb[seg], n0, g.N, k0, g.b_rows[seg], wid, lane);
  };
  if (nit > 0) issue(0, A0, B0);
  wait_loads();
  __syncthreads();
  int64_t it = 0;
  for (; it + 1 < nit; it += 2) {
    issue(it + 1, A1, B1);
    mma_stage<AKC, BKC>(A0, B0, acc, lane, abase, bbase);
    wait_loads();
    __syncthreads();
    if (it + 2 < nit) issue(it + 2, A0, B0);
    mma_stage<AKC, BKC>(A1, B1, acc, lane, abase, bbase);
    wait_loads();
    __syncthreads();
  }
  if (it < nit) mma_stage<AKC, BKC>(A0, B0, acc, lane, abase, bbase);  // odd block count

  // ---------------------------------------------------------------- epilogues
  // The lane indices are re-read through an empty asm so that no epilogue
  // address is computed before the loop and kept live across it.
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));

  const int i16e = lane_e & 15, g4e = lane_e >> 4;
  const int64_t rbase = m0 + wm * WM + 4 * g4e;  // + 16 i + r
  const int64_t cbase = n0 + wn * WN + i16e;     // + 16 j
  float* red = (float*)smem;
  __syncthreads();  // every wave is done with the operand tiles
  lu16* const T = A0 + wid * EP_ELEMS;  // this wave's staging region
  const int64_t wrow0 = m0 + wm * WM;    // this wave's first row

  if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_H) {
    // Columns are interleaved in blocks of 64: [G of 32 units | U of the same
    // 32]; a wave holds one such block (G in column tiles 0-1, U in 2-3).
    const int64_t hid0 = ((n0 + wn * WN) >> 6) * 32;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float hv[4], av[4], gv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gg = acc[i][j][r], uu = acc[i][j + 2][r];
          const float s = sigmoid_fast(gg);
          const float a = gg * s;
          const float h = a * uu;
          // Rows past M (up to the tile boundary) are stored as zeros: the
          // token-reduction GEMMs read them as the zero operand of their tail.
          hv[r] = rbase + 16 * i + r < g.M ? h : 0.0f;
          av[r] = a;
          gv[r] = fmaf(-h, s, fmaf(uu, s, h));
        }
        ep_put(T, i, j, i16e, g4e, hv[0], hv[1], hv[2], hv[3]);
        if constexpr (EPI == EPI_SWIGLU) {
          const int64_t o = cn_off(wrow0 + 16 * i, hid0 + 16 * j, g.ldo, lane_e);
          st8(g.out1 + o, u32x2{pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3])});
          st8(g.out2 + o, u32x2{pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3])});
        }
      }
    }
    ep_flush<4>(T, g.out0, g.ldo, wrow0, hid0, EPI == EPI_SWIGLU ? wrow0 + 128 : g.M, lane_e);
  } else if constexpr (EPI == EPI_Y_LOSS || EPI == EPI_Y_STORE) {
    float loss = 0.0f;
    if constexpr (EPI == EPI_Y_LOSS) {
      // V' for this wave's 128 x 64 outputs: 16-byte loads into LDS (row-major),
      // then one transpose read per 16x16 tile gives each lane its 4 rows.
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int qd = it * 64 + lane_e, r = qd >> 3, cc = qd & 7;
        int64_t row = wrow0 + r;
        row = row < g.M ? row : g.M - 1;
        const u32x4 v = ld16(g.in0 + row * g.ldi + n0 + wn * WN + 8 * cc);
        *(lu32x4*)(T + r * VP_P + 8 * cc) = v;
      }
      const int jr4 = i16e >> 2, q4e = i16e & 3;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const u32x2 vv = ltr(T + (16 * i + 4 * g4e + jr4) * VP_P + 16 * j + 4 * q4e);
          const float v[4] = {bf16_lo(vv[0]), bf16_hi(vv[0]), bf16_lo(vv[1]), bf16_hi(vv[1])};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float rr = acc[i][j][r] - v[r];
            if (rbase + 16 * i + r < g.M) loss = fmaf(rr, rr, loss);
          }
        }
      }
    }
    const float sg = EPI == EPI_Y_LOSS ? -1.0f : 1.0f;  // P2 stores -Y
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        ep_put(T, i, j, i16e, g4e, sg * acc[i][j][0], sg * acc[i][j][1], sg * acc[i][j][2], sg * acc[i][j][3]);
    ep_flush<8>(T, g.out0, g.ldo, wrow0, n0 + wn * WN, g.M, lane_e);
    if constexpr (EPI == EPI_Y_LOSS) {
      const float s = block_sum(loss, red, tid);
      if (tid == 0) g.fout[t] = s;
    }
  } else if constexpr (EPI == EPI_DH) {
    // [dG | dU] = [D * GP | D * A], rows past M stored as zeros (see EPI_SWIGLU).
    float dv[TM][TN][4];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t o = cn_off(wrow0 + 16 * i, n0 + wn * WN + 16 * j, g.N, lane_e);
        const u32x2 ap = ld8(g.in1 + o), gp = ld8(g.in0 + o);
        const float av[4] = {bf16_lo(ap[0]), bf16_hi(ap[0]), bf16_lo(ap[1]), bf16_hi(ap[1])};
        const float gv[4] = {bf16_lo(gp[0]), bf16_hi(gp[0]), bf16_lo(gp[1]), bf16_hi(gp[1])};
        float dg[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float dh = rbase + 16 * i + r < g.M ? acc[i][j][r] : 0.0f;
          dg[r] = dh * gv[r];
          dv[i][j][r] = dh * av[r];
        }
        ep_put(T, i, j, i16e, g4e, dg[0], dg[1], dg[2], dg[3]);
      }
    }
    ep_flush<8>(T, g.out0, g.ldo, wrow0, n0 + wn * WN, wrow0 + 128, lane_e);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) ep_put(T, i, j, i16e, g4e, dv[i][j][0], dv[i][j][1], dv[i][j][2], dv[i][j][3]);
    ep_flush<8>(T, g.out0 + g.N, g.ldo, wrow0, n0 + wn * WN, wrow0 + 128, lane_e);
  } else if constexpr (EPI == EPI_PARTIAL) {
    float* dst = g.fout + (int64_t)slice * g.M * g.N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t o = cn_off(m0 + wm * WM + 16 * i, n0 + wn * WN + 16 * j, g.N, lane_e);
        f32x4 v = acc[i][j];
        if (g.accumulate) v += *(const f32x4*)(dst + o);
        *(f32x4*)(dst + o) = v;
      }
    }
  }
}

template <bool AKC, bool BKC, int EPI>
hipError_t launch_t(const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles = ((g.M + BM - 1) / BM) * (g.N / BN);
  hipLaunchKernelGGL((gemm_kernel<AKC, BKC, EPI>), dim3((unsigned)(tiles * g.S)), dim3(NTHR), 0, stream, g);
  return hipGetLastError();
}

// ------------------------------------------------------------ weight packing
// theta (fp32, per head [W_g d x m | W_u d x m | W_d m x d]) -> bf16 GEMM operands:
//   wgu [2m][d]: row 64b + q is column 32b + q of W_g (q < 32) or column
//                32b + q - 32 of W_u (q >= 32), i.e. [W_g | W_u]^T interleaved
//                in blocks of 32 hidden units;
//   wdt [d][m]:  W_d^T;
//   wdn [m][d]:  W_d.
__global__ __launch_bounds__(256) void pack_gu_kernel(const float* __restrict__ theta, uint16_t* __restrict__ wgu,
                                                      int d, int m) {
  __shared__ float tile[64][65];
  const int jb = blockIdx.x;          // 64 packed rows = hidden units 32jb .. 32jb+31 of W_g and W_u
  const int k0 = blockIdx.y * 64;
  const int64_t dm = (int64_t)d * m;
  for (int idx = threadIdx.x; idx < 64 * 64; idx += 256) {
    const int kk = idx >> 6, q = idx & 63;
    const int h = 32 * jb + (q & 31);
    tile[q][kk] = theta[(q >> 5) * dm + (int64_t)(k0 + kk) * m + h];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 64 * 64; idx += 256) {
    const int q = idx >> 6, kk = idx & 63;
    wgu[(int64_t)(64 * jb + q) * d + k0 + kk] = f32_to_bf16_bits(tile[q][kk]);
  }
}

__global__ __launch_bounds__(256) void pack_d_kernel(const float* __restrict__ theta, uint16_t* __restrict__ wdt,
                                                     uint16_t* __restrict__ wdn, int d, int m) {
  __shared__ float tile[64][65];
  const int h0 = blockIdx.x * 64, o0 = blockIdx.y * 64;
  const float* wd = theta + 2 * (int64_t)d * m;
  for (int idx = threadIdx.x; idx < 64 * 64; idx += 256) {
    const int hh = idx >> 6, oo = idx & 63;
    const float v = wd[(int64_t)(h0 + hh) * d + o0 + oo];
    tile[oo][hh] = v;
    wdn[(int64_t)(h0 + hh) * d + o0 + oo] = f32_to_bf16_bits(v);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 64 * 64; idx += 256) {
    const int oo = idx >> 6, hh = idx & 63;
    wdt[(int64_t)(o0 + oo) * m + h0 + hh] = f32_to_bf16_bits(tile[oo][hh]);
  }
}

// ----------------------------------------------------- gradient reduction
// Sum the S split-K partials (fixed pairwise tree) of the two gradient GEMMs
// (C-native [d x 2m] = [gW_g | gW_u] and [m x d] = gW_d), scale, and apply to
// theta / store / accumulate into grad in theta layout.
// With wd_dot != NULL each block also writes, to wd_dot[block], the sum over
// its W_d elements of theta_old * g (theta read before any update).
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ p_gu,
                                                              const float* __restrict__ p_d, int S, int d, int m,
                                                              float scale, int mode, float* __restrict__ dst,
                                                              float lr, const float* __restrict__ theta,
                                                              float* __restrict__ wd_dot) {
  __shared__ float red[4];
  const int64_t n_gu = 2 * (int64_t)d * m, n_all = 3 * (int64_t)d * m;
  const int64_t dm = (int64_t)d * m;
  float dotv = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_all; i += (int64_t)gridDim.x * 256) {
    const bool gu = i < n_gu;
    const int64_t ci = gu ? i : i - n_gu;
    const float* p = gu ? p_gu : p_d;
    const int64_t stride = gu ? n_gu : dm;
    float v[16];
    for (int s = 0; s < S; ++s) v[s] = p[(int64_t)s * stride + ci];
    for (int w = 1; w < S; w <<= 1)
      for (int s = 0; s + w < S; s += 2 * w) v[s] += v[s + w];
    const float gsum = v[0] * scale;
    // C-native index -> (row, col)
    const int64_t blk = ci >> 8;
    const int within = (int)(ci & 255);
    const int l = within >> 2, r = within & 3;
    const int64_t ncol = gu ? 2 * (int64_t)m : d;
    const int64_t row = (blk / (ncol >> 4)) * 16 + 4 * (l >> 4) + r;
    const int64_t col = (blk % (ncol >> 4)) * 16 + (l & 15);
    int64_t ti;
    if (gu)
      ti = col < m ? row * m + col : dm + row * m + (col - m);
    else
      ti = 2 * dm + row * d + col;
    if (wd_dot != nullptr && !gu) dotv = fmaf(theta[ti], gsum, dotv);
    if (mode == kApply)
      dst[ti] -= lr * gsum;
    else if (mode == kStore)
      dst[ti] = gsum;
    else
      dst[ti] += gsum;
  }
  if (wd_dot != nullptr) {
    dotv = wave_sum(dotv);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = dotv;
    __syncthreads();
    if (threadIdx.x == 0) wd_dot[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
  }
}

// Fixed-order sum of n loss partials (one workgroup): out = scale * sum, or
// out += scale * sum.
__global__ __launch_bounds__(256) void sum_kernel(const float* __restrict__ x, int64_t n, float scale, int accumulate,
                                                  float* __restrict__ out) {
  __shared__ float red[4];
  float s = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += x[i];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float v = ((red[0] + red[1]) + (red[2] + red[3])) * scale;
    *out = accumulate ? *out + v : v;
  }
}

}  // namespace

hipError_t launch_gemm(int kind, const GemmArgs& g, hipStream_t stream) {
  switch (kind) {
    case EPI_SWIGLU: return launch_t<true, true, EPI_SWIGLU>(g, stream);
    case EPI_SWIGLU_H: return launch_t<true, true, EPI_SWIGLU_H>(g, stream);
    case EPI_Y_LOSS: return launch_t<true, true, EPI_Y_LOSS>(g, stream);
    case EPI_Y_STORE: return launch_t<true, true, EPI_Y_STORE>(g, stream);
    case EPI_DH: return launch_t<true, true, EPI_DH>(g, stream);
    case EPI_PARTIAL: return launch_t<false, false, EPI_PARTIAL>(g, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pack(const float* theta, uint16_t* wgu, uint16_t* wdt, uint16_t* wdn, int d, int m,
                       hipStream_t stream) {
  hipLaunchKernelGGL(pack_gu_kernel, dim3(2 * m / 64, d / 64), dim3(256), 0, stream, theta, wgu, d, m);
  hipLaunchKernelGGL(pack_d_kernel, dim3(m / 64, d / 64), dim3(256), 0, stream, theta, wdt, wdn, d, m);
  return hipGetLastError();
}

hipError_t launch_reduce_partials(const float* p_gu, const float* p_d, int S, int d, int m, float scale, int mode,
                                  float* dst, float lr, const float* theta, float* wd_dot, hipStream_t stream) {
  hipLaunchKernelGGL(reduce_partials_kernel, dim3(reduce_blocks(d, m)), dim3(256), 0, stream, p_gu, p_d, S, d, m,
                     scale, mode, dst, lr, theta, wd_dot);
  return hipGetLastError();
}

hipError_t launch_sum(const float* x, int64_t n, float scale, int accumulate, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(sum_kernel, dim3(1), dim3(256), 0, stream, x, n, scale, accumulate, out);
  return hipGetLastError();
}

}  // namespace wide
}  // namespace vggt3

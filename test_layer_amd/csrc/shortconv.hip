// ShortConv2D on the value tokens: depthwise 3x3 over each view's patch grid.
//
// Paper-graph summary "VGG-T3: Offline Feed-Forward 3D Reconstruction at Scale",
// section 3.4 "Non-Linear Spatial Mixing via ShortConv2D": the value tokens of a
// view are put back on their (H/p, W/p) patch grid, mixed by one 3x3 conv and
// flattened again; per its Appendix A note, camera and register tokens bypass
// the conv. The conv is depthwise (one 3x3 filter per channel), zero padded.
//
// Design (HBM-bound stencil). Two kernels share one arithmetic contract.
//
// shortconv_lds_kernel<CB, R, NT> (bf16, 3x3, channels a multiple of 64, grid
// rows up to 126 columns): an LDS-haloed stencil. A workgroup walks strips
// (view, block of CB channels) down the grid in blocks of R output rows. LDS
// holds a ring of 2R + 4 staged input rows [slot][column][CB channels] (bf16,
// 2 CB bytes per token) with a zero column on each side; every block brings in
// the rows it needs that are not staged yet (a strip's first block: the zero
// row above the grid and rows 0..R; later blocks: the next R rows, or the zero
// row below the grid) with direct global -> LDS loads (global_load_lds_dwordx4,
// one 64-lane instruction per 1 KB of a row), so each input row is read from
// HBM once. Those loads for block k + 1 are issued before block k is computed
// and fill ring slots block k does not read: one barrier per block, and the
// loads overlap the arithmetic. Thread (q, x) computes channel quad q of column
// x with a rotating 3x3 window of LDS reads; CB / 4 lanes cover a token's
// 2 CB bytes, so LDS reads and the output stores are contiguous. The grid is a
// multiple of the channel-block count, so a workgroup's strips share one
// channel block and it loads its filters once. 128-channel strips (256
// contiguous bytes per token and access) are used where C allows and the ring
// fits, 64-channel strips otherwise.
//
// shortconv_kernel (everything else: fp32, wider grids, other channel counts):
// a work item is one (view, column x, segment of SEG rows, block of up to 256
// 4-channel groups); a few workgroups per CU walk the items with a grid stride
// (loading the filters once), and thread t owns channel group 256*block + t.
// Everything that decides which taps exist (x at a grid edge, the segment
// touching the top or bottom row) is therefore uniform across the workgroup:
// the left/right edges select a template instance, and rows outside the grid
// become scalar branches that skip those taps instead of selecting zeros per
// element. Each thread issues the loads of all SEG+2 input rows of its segment
// at columns x-1, x, x+1 at once (8 bytes each; about 23 KB in flight per
// wave) from a uniform row address plus its 32-bit lane offset, then computes
// the SEG output rows with a rotating 3x3 window of fp32 vectors in registers.
// Lanes of a wave cover consecutive channel groups of one token (512 contiguous
// bytes per wave access); the x-1 / x+1 re-reads of neighbouring columns hit
// L1/L2, and workgroups are remapped so that each XCD walks a contiguous range
// of columns.
//
// Bit-exact contract: acc = +0; taps with the row offset outermost and the
// column offset innermost; acc = fl(acc + fl(w*v)), never fused (this file is
// compiled with -ffp-contract=off and the pragma below); out-of-grid taps see
// v = 0; the result is rounded to bf16 with ties to even. An out-of-grid tap
// adds fl(w*0) = +-0 to an accumulator that is never -0 (it starts at +0 and a
// round-to-nearest sum is -0 only if both terms are), which leaves it
// unchanged, so shortconv_kernel skips such taps and shortconv_lds_kernel
// multiplies the staged zeros: both give the same bits for finite filters.
#include "common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace vggt3 {

namespace {

#ifndef VGGT3_CONV_WG_PER_CU
#define VGGT3_CONV_WG_PER_CU 8
#endif
#ifndef VGGT3_CONV_SEG
#define VGGT3_CONV_SEG 13
#endif
constexpr int SEG = VGGT3_CONV_SEG;  // output rows per thread (37 rows -> 3 segments)
constexpr int MAX_W = 4096;  // widest grid row accepted (no staging limit in this design)

template <bool BF16>
struct ConvTraits;
template <>
struct ConvTraits<true> {
  static constexpr int ESZ = 2;
  typedef u32x2 vec_t;  // 4 bf16
  __device__ static void widen(const vec_t& q, float (&v)[4]) {
    v[0] = bf16_lo(q[0]);
    v[1] = bf16_hi(q[0]);
    v[2] = bf16_lo(q[1]);
    v[3] = bf16_hi(q[1]);
  }
  __device__ static vec_t narrow(const float (&v)[4]) {
    return vec_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
};
template <>
struct ConvTraits<false> {
  static constexpr int ESZ = 4;
  typedef u32x4 vec_t;  // 4 fp32
  __device__ static void widen(const vec_t& q, float (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(q[i]);
  }
  __device__ static vec_t narrow(const float (&v)[4]) {
    return vec_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
  }
};

// Output rows [y0, y0 + SEG) of one column for one channel group. HAS_L /
// HAS_R: whether columns x-1 / x+1 exist. `in_col` points at (y = 0, x) of the
// input patch grid, `out_col` likewise; `lane` is this thread's byte offset in
// a token row; `row_bytes` is one token row, `grid_row` one patch-grid row.
template <bool BF16, bool HAS_L, bool HAS_R>
__device__ __forceinline__ void conv_segment(const char* in_col, char* out_col, uint32_t lane,
                                             int64_t row_bytes, int64_t grid_row, int y0, int grid_h,
                                             const float (&wt)[9][4]) {
  using Tr = ConvTraits<BF16>;
  typedef typename Tr::vec_t vec_t;
  // All SEG+2 input rows, from in-grid (clamped) addresses; rows outside the
  // grid are loaded but never used.
  vec_t raw[SEG + 2][3];
#pragma unroll
  for (int k = 0; k < SEG + 2; ++k) {
    const int y = y0 - 1 + k;
    const int yc = y < 0 ? 0 : (y >= grid_h ? grid_h - 1 : y);
    const char* p = in_col + (int64_t)yc * grid_row;
    if (HAS_L) raw[k][0] = *reinterpret_cast<const vec_t*>(p - row_bytes + lane);
    raw[k][1] = *reinterpret_cast<const vec_t*>(p + lane);
    if (HAS_R) raw[k][2] = *reinterpret_cast<const vec_t*>(p + row_bytes + lane);
  }
  float win[3][3][4];  // widened rows, rotating: win[k % 3] holds input row y0 - 1 + k
  auto widen_row = [&](int k) {
#pragma unroll
    for (int b = 0; b < 3; ++b)
      if ((b != 0 || HAS_L) && (b != 2 || HAS_R)) Tr::widen(raw[k][b], win[k % 3][b]);
  };
  auto taps = [&](int a, int k, float (&acc)[4]) {  // row offset a (0..2) from window row k
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      if ((b == 0 && !HAS_L) || (b == 2 && !HAS_R)) continue;
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) acc[ch] = acc[ch] + wt[3 * a + b][ch] * win[k % 3][b][ch];
    }
  };
  widen_row(0);
  widen_row(1);
#pragma unroll
  for (int k = 0; k < SEG; ++k) {
    widen_row(k + 2);
    const int y = y0 + k;
    if (y >= grid_h) break;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (y > 0) taps(0, k, acc);
    taps(1, k + 1, acc);
    if (y + 1 < grid_h) taps(2, k + 2, acc);
    // V' is not read again by this kernel: stream it past the caches, which
    // keeps them for the input rows that neighbouring columns re-read.
    __builtin_nontemporal_store(Tr::narrow(acc), reinterpret_cast<vec_t*>(out_col + (int64_t)y * grid_row + lane));
  }
}

// Work item = (view, segment, column x, channel block), channel block fastest,
// so consecutive workgroups read neighbouring columns of one segment.
template <bool BF16>
__global__ __launch_bounds__(256) void shortconv_kernel(const char* __restrict__ V, char* __restrict__ Vp,
                                                         const float* __restrict__ w, int64_t n_work,
                                                         int grid_h, int grid_w, int n_special, int C,
                                                         int n_seg, int n_cblk) {
  using Tr = ConvTraits<BF16>;
  typedef typename Tr::vec_t vec_t;
  constexpr int VB = (int)sizeof(vec_t);  // bytes per 4-channel group
  const int CG = C / 4;
  const int64_t row_bytes = (int64_t)C * Tr::ESZ;
  const int64_t tpv = (int64_t)n_special + (int64_t)grid_h * grid_w;
  const int64_t grid_row = (int64_t)grid_w * row_bytes;
  const int64_t stride = gridDim.x;
  float wt[9][4];
  int wt_cblk = -1;
  for (int64_t wi = xcd_remap(blockIdx.x, stride); wi < n_work; wi += stride) {
    const int cblk = (int)(wi % n_cblk);
    int64_t rest = wi / n_cblk;
    const int x = (int)(rest % grid_w);
    rest /= grid_w;
    const int seg = (int)(rest % n_seg);
    const int64_t view = rest / n_seg;
    const int cg = cblk * 256 + (int)threadIdx.x;
    if (cg >= CG) continue;
    const uint32_t lane = (uint32_t)cg * VB;
    const char* vview = V + view * tpv * row_bytes;
    char* oview = Vp + view * tpv * row_bytes;

    if (x == 0 && seg == 0) {
      for (int s = 0; s < n_special; ++s)
        *reinterpret_cast<vec_t*>(oview + s * row_bytes + lane) =
            *reinterpret_cast<const vec_t*>(vview + s * row_bytes + lane);
    }

    if (cblk != wt_cblk) {  // the filters of this channel block, loaded once per block change
#pragma unroll
      for (int ch = 0; ch < 4; ++ch)
#pragma unroll
        for (int t = 0; t < 9; ++t) wt[t][ch] = w[(int64_t)(cg * 4 + ch) * 9 + t];
      wt_cblk = cblk;
    }

    const int64_t col = ((int64_t)n_special + x) * row_bytes;
    const char* in_col = vview + col;
    char* out_col = oview + col;
    const int y0 = seg * SEG;
    const bool has_l = x > 0, has_r = x + 1 < grid_w;
    if (has_l && has_r)
      conv_segment<BF16, true, true>(in_col, out_col, lane, row_bytes, grid_row, y0, grid_h, wt);
    else if (has_l)
      conv_segment<BF16, true, false>(in_col, out_col, lane, row_bytes, grid_row, y0, grid_h, wt);
    else if (has_r)
      conv_segment<BF16, false, true>(in_col, out_col, lane, row_bytes, grid_row, y0, grid_h, wt);
    else
      conv_segment<BF16, false, false>(in_col, out_col, lane, row_bytes, grid_row, y0, grid_h, wt);
  }
}

// Any odd k x k filter (the pages' "V-5" variant of Table 9 uses k = 5): the
// same work items and contract (row offset outer, column offset inner, both
// -k/2..k/2, separately rounded fp32 product and sum, out-of-grid taps
// skipped). A thread owns SEGK output rows; it keeps its channel group's
// k*k filters in registers, issues the loads of all SEGK + k - 1 input rows at
// the k columns at once (clamped, in-grid addresses; taps outside the grid are
// skipped by uniform branches), and widens each row's taps as it needs them.
constexpr int SEGK = 4;

template <bool BF16, int KS>
__global__ __launch_bounds__(256) void shortconv_kxk_kernel(const char* __restrict__ V, char* __restrict__ Vp,
                                                             const float* __restrict__ w, int64_t n_work,
                                                             int grid_h, int grid_w, int n_special, int C,
                                                             int n_seg, int n_cblk) {
  using Tr = ConvTraits<BF16>;
  typedef typename Tr::vec_t vec_t;
  constexpr int VB = (int)sizeof(vec_t);
  constexpr int R = KS / 2;
  constexpr int NR = SEGK + KS - 1;  // input rows per segment
  const int CG = C / 4;
  const int64_t row_bytes = (int64_t)C * Tr::ESZ;
  const int64_t tpv = (int64_t)n_special + (int64_t)grid_h * grid_w;
  const int64_t grid_row = (int64_t)grid_w * row_bytes;
  const int64_t stride = gridDim.x;
  float wt[KS * KS][4];
  int wt_cblk = -1;
  for (int64_t wi = xcd_remap(blockIdx.x, stride); wi < n_work; wi += stride) {
    const int cblk = (int)(wi % n_cblk);
    int64_t rest = wi / n_cblk;
    const int x = (int)(rest % grid_w);
    rest /= grid_w;
    const int seg = (int)(rest % n_seg);
    const int64_t view = rest / n_seg;
    const int cg = cblk * 256 + (int)threadIdx.x;
    if (cg >= CG) continue;
    const uint32_t lane = (uint32_t)cg * VB;
    const char* vview = V + view * tpv * row_bytes;
    char* oview = Vp + view * tpv * row_bytes;
    if (x == 0 && seg == 0) {
      for (int s = 0; s < n_special; ++s)
        *reinterpret_cast<vec_t*>(oview + s * row_bytes + lane) =
            *reinterpret_cast<const vec_t*>(vview + s * row_bytes + lane);
    }
    if (cblk != wt_cblk) {
#pragma unroll
      for (int ch = 0; ch < 4; ++ch)
#pragma unroll
        for (int t = 0; t < KS * KS; ++t) wt[t][ch] = w[(int64_t)(cg * 4 + ch) * KS * KS + t];
      wt_cblk = cblk;
    }
    const char* in_col = vview + ((int64_t)n_special + x) * row_bytes;
    char* out_col = oview + ((int64_t)n_special + x) * row_bytes;
    const int y0 = seg * SEGK;
    vec_t raw[NR][KS];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int y = y0 - R + k;
      const int yc = y < 0 ? 0 : (y >= grid_h ? grid_h - 1 : y);
      const char* p = in_col + (int64_t)yc * grid_row + lane;
#pragma unroll
      for (int b = 0; b < KS; ++b) {
        const int xc = x + b - R < 0 ? -x : (x + b - R >= grid_w ? grid_w - 1 - x : b - R);
        raw[k][b] = *reinterpret_cast<const vec_t*>(p + xc * row_bytes);
      }
    }
#pragma unroll
    for (int k = 0; k < SEGK; ++k) {
      const int y = y0 + k;
      if (y >= grid_h) break;
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int a = 0; a < KS; ++a) {
        if (y + a - R < 0 || y + a - R >= grid_h) continue;
#pragma unroll
        for (int b = 0; b < KS; ++b) {
          if (x + b - R < 0 || x + b - R >= grid_w) continue;
          float v[4];
          Tr::widen(raw[k + a][b], v);
#pragma unroll
          for (int ch = 0; ch < 4; ++ch) acc[ch] = acc[ch] + wt[a * KS + b][ch] * v[ch];
        }
      }
      __builtin_nontemporal_store(Tr::narrow(acc), reinterpret_cast<vec_t*>(out_col + (int64_t)y * grid_row + lane));
    }
  }
}


// ---------------------------------------------------------------------------
// LDS-haloed form (bf16, 3x3); see the file header.
// Two shapes of the ring, as template parameters <CB channels per strip, R
// output rows per block, NT threads>:
//   <128, 2, 512>: 256 bytes per token and strip, 8 slots (79.9 KB at 37
//     columns), two workgroups per CU; used when C is a multiple of 128 and
//     the ring fits.
//   <64, 3, 256>: 128 bytes per token, 10 slots (49.9 KB at 37 columns), three
//     workgroups per CU; every other bf16 case with C a multiple of 64.
constexpr size_t LDS_MAX_BYTES = 160 * 1024;
template <int CB, int R>
constexpr size_t lds_ring_bytes(int grid_w) {
  return (size_t)(2 * R + 4) * (grid_w + 2) * CB * 2;
}

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) void lds_void;

// Ring bookkeeping: each block "introduces" rows into the next free slots (in
// order). Block 0 of a strip introduces the zero row -1 and rows 0 .. R (R + 2
// slots), block b > 0 rows bR+1 .. bR+R (R slots; rows past the grid are not
// loaded, and the row just below the grid is zeroed when it is among them).
// A block's R + 2 input rows bR-1 .. bR+R are then consecutive slots starting
// at `start` (its first introduced slot for b = 0, two before it otherwise);
// the next block's rows go to the R + 2 slots after them, which this block does
// not read. That needs 2R + 4 slots.
template <int CB, int R, int NT>
__global__ __launch_bounds__(NT) void shortconv_lds_kernel(const uint16_t* __restrict__ V,
                                                              uint16_t* __restrict__ Vp, const float* __restrict__ w,
                                                              int64_t n_strips, int grid_h, int grid_w, int n_special,
                                                              int C, int n_cb, int pieces_per_row) {
  extern __shared__ __attribute__((aligned(16))) uint16_t ring[];
  constexpr int NS = 2 * R + 4;  // ring slots
  constexpr int NQ = CB / 4;   // 4-channel quads per token
  constexpr int NCH = CB / 8;  // 16-byte chunks per token
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int W2 = grid_w + 2;
  const int row_chunks = grid_w * NCH;
  const int n_blk = (grid_h + R - 1) / R;
  const int64_t tpv = (int64_t)n_special + (int64_t)grid_h * grid_w;
  const int64_t G = gridDim.x;
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  for (int i = tid; i < NS * 2 * NCH; i += NT) {  // the side columns of every slot stay zero
    const int slot = i / (2 * NCH), side = (i / NCH) & 1, c = i % NCH;
    *reinterpret_cast<u32x4*>(ring + (slot * W2 + (side ? W2 - 1 : 0)) * CB + 8 * c) = z4;
  }

  auto introduce = [&](int64_t strip, int b, int first) {
    const int cb = (int)(strip % n_cb);
    const int64_t tok0 = (strip / n_cb) * tpv;
    if (b == 0) {  // special tokens pass through (before any direct load is in flight)
      for (int i = tid; i < n_special * NCH; i += NT) {
        const int64_t o = (tok0 + i / NCH) * C + (int64_t)cb * CB + 8 * (i % NCH);
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(V + o), reinterpret_cast<u32x4*>(Vp + o));
      }
    }
    const int y_new = b == 0 ? 0 : b * R + 1;
    const int want = b == 0 ? R + 1 : R;
    int n_new = grid_h - y_new < want ? grid_h - y_new : want;
    if (n_new < 0) n_new = 0;
    int s_new = b == 0 ? first + 1 : first;  // slot of row y_new
    if (s_new >= NS) s_new -= NS;
    const uint16_t* src = V + (tok0 + n_special + (int64_t)y_new * grid_w) * C + (int64_t)cb * CB;
    // wave instruction i of n_new * pieces_per_row loads piece i % ppr (64 chunks) of row i / ppr
    int row = 0, k = wid;
    while (k >= pieces_per_row) {
      k -= pieces_per_row;
      ++row;
    }
    while (row < n_new) {
      int slot = s_new + row;
      if (slot >= NS) slot -= NS;
      const int j = k * 64 + lane;  // chunk of the row: token j / NCH, 16-byte part j % NCH
      if (j < row_chunks) {
        const uint16_t* g = src + ((int64_t)row * grid_w + j / NCH) * C + 8 * (j % NCH);
        __builtin_amdgcn_global_load_lds(g, (lds_void*)((lds_u16*)ring + (slot * W2 + 1) * CB + k * 512), 16, 0,
                                         0);
      }
      k += NW;
      while (k >= pieces_per_row) {
        k -= pieces_per_row;
        ++row;
      }
    }
    if (b == 0)  // row -1
      for (int i = tid; i < row_chunks; i += NT) *reinterpret_cast<u32x4*>(ring + (first * W2 + 1) * CB + 8 * i) = z4;
    if (grid_h >= y_new && grid_h < y_new + want) {  // row grid_h
      int slot = s_new + (grid_h - y_new);
      if (slot >= NS) slot -= NS;
      for (int i = tid; i < row_chunks; i += NT) *reinterpret_cast<u32x4*>(ring + (slot * W2 + 1) * CB + 8 * i) = z4;
    }
  };

  int64_t s_cur = xcd_remap(blockIdx.x, G);
  if (s_cur >= n_strips) return;
  const int q = tid % NQ;
  float wt[9][4];
  {
    const int cb = (int)(s_cur % n_cb);  // the same for all strips s_cur + k G
#pragma unroll
    for (int t = 0; t < 9; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) wt[t][j] = w[(int64_t)(cb * CB + 4 * q + j) * 9 + t];
  }

  auto compute = [&](int64_t strip, int b, int start) {
    const int cb = (int)(strip % n_cb);
    const int y0 = b * R;
    const int rows = grid_h - y0 < R ? grid_h - y0 : R;
    uint16_t* ob = Vp + ((strip / n_cb) * tpv + n_special + (int64_t)y0 * grid_w) * C + (int64_t)cb * CB + 4 * q;
    for (int x = tid / NQ; x < grid_w; x += NT / NQ) {
      const uint16_t* col = ring + x * CB + 4 * q;  // staged column x holds input column x - 1
      float win[3][3][4];  // win[k % 3][dx]: input row y0 - 1 + k, columns x - 1 .. x + 1
      auto fetch = [&](int k, int dst) {
        int slot = start + k;
        if (slot >= NS) slot -= NS;
#pragma unroll
        for (int dx = 0; dx < 3; ++dx)
          ConvTraits<true>::widen(*reinterpret_cast<const u32x2*>(col + (slot * W2 + dx) * CB), win[dst][dx]);
      };
      fetch(0, 0);
      fetch(1, 1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r >= rows) break;
        fetch(r + 2, (r + 2) % 3);
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int dy = 0; dy < 3; ++dy)
#pragma unroll
          for (int dx = 0; dx < 3; ++dx)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float p = wt[3 * dy + dx][j] * win[(r + dy) % 3][dx][j];
              acc[j] = acc[j] + p;
            }
        __builtin_nontemporal_store(ConvTraits<true>::narrow(acc),
                                    reinterpret_cast<u32x2*>(ob + ((int64_t)r * grid_w + x) * C));
      }
    }
  };

  int b_cur = 0, first_cur = 0;
  introduce(s_cur, 0, first_cur);
  int first_next = R + 2;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  while (true) {
    int64_t s_next = s_cur;
    int b_next = b_cur + 1;
    if (b_next == n_blk) {
      b_next = 0;
      s_next = s_cur + G;
    }
    const bool more = s_next < n_strips;
    if (more) introduce(s_next, b_next, first_next);
    compute(s_cur, b_cur, b_cur == 0 ? first_cur : (first_cur + NS - 2) % NS);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's direct loads have landed
    __syncthreads();
    if (!more) break;
    first_cur = first_next;
    first_next = (first_next + (b_next == 0 ? R + 2 : R)) % NS;
    s_cur = s_next;
    b_cur = b_next;
  }
}


// Launches the LDS ring kernel with a grid that is a multiple of the channel
// block count, so that the strips s, s + G, ... of a workgroup share a channel
// block. False (and nothing launched) if the ring needs more dynamic LDS than
// the device grants.
template <int CB, int R, int NT>
bool launch_lds(const void* V, void* Vp, const float* w, int64_t n_views, int grid_h, int grid_w, int n_special,
                int C, int wg_per_cu, hipStream_t stream) {
  const size_t ring_bytes = lds_ring_bytes<CB, R>(grid_w);
  if (ring_bytes > 64 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(&shortconv_lds_kernel<CB, R, NT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)ring_bytes) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  const int n_cb = C / CB;
  const int64_t n_strips = n_views * n_cb;
  int64_t g = (int64_t)wg_per_cu * 256 / n_cb;
  g = (g < 1 ? 1 : g) * n_cb;
  if (g > n_strips) g = n_strips;
  const int pieces_per_row = (grid_w * (CB / 8) + 63) / 64;
  hipLaunchKernelGGL((shortconv_lds_kernel<CB, R, NT>), dim3((unsigned)g), dim3(NT), ring_bytes, stream,
                     static_cast<const uint16_t*>(V), static_cast<uint16_t*>(Vp), w, n_strips, grid_h, grid_w,
                     n_special, C, n_cb, pieces_per_row);
  return true;
}

}  // namespace

hipError_t launch_shortconv_k(const void* V, void* Vp, const float* w, int64_t n_views, int grid_h, int grid_w,
                              int n_special, int C, int ksize, bool bf16, hipStream_t stream) {
  if (ksize == 3) return launch_shortconv(V, Vp, w, n_views, grid_h, grid_w, n_special, C, bf16, stream);
  if (ksize != 5) return hipErrorInvalidValue;
  const int n_seg = (grid_h + SEGK - 1) / SEGK;
  const int n_cblk = (C / 4 + 255) / 256;
  const int64_t n_work = n_views * grid_w * (int64_t)n_seg * n_cblk;
  if (n_work == 0) return hipSuccess;
  const int64_t max_grid = (int64_t)VGGT3_CONV_WG_PER_CU * 256;
  const unsigned n_blocks = (unsigned)(n_work < max_grid ? n_work : max_grid);
  if (bf16)
    hipLaunchKernelGGL((shortconv_kxk_kernel<true, 5>), dim3(n_blocks), dim3(256), 0, stream,
                       static_cast<const char*>(V), static_cast<char*>(Vp), w, n_work, grid_h, grid_w, n_special, C,
                       n_seg, n_cblk);
  else
    hipLaunchKernelGGL((shortconv_kxk_kernel<false, 5>), dim3(n_blocks), dim3(256), 0, stream,
                       static_cast<const char*>(V), static_cast<char*>(Vp), w, n_work, grid_h, grid_w, n_special, C,
                       n_seg, n_cblk);
  return hipGetLastError();
}

hipError_t launch_shortconv(const void* V, void* Vp, const float* w, int64_t n_views, int grid_h,
                            int grid_w, int n_special, int C, bool bf16, hipStream_t stream) {
  const int n_seg = (grid_h + SEG - 1) / SEG;
  const int n_cblk = (C / 4 + 255) / 256;
  const int64_t n_work = n_views * grid_w * (int64_t)n_seg * n_cblk;
  if (n_work == 0) return hipSuccess;
  // A few resident workgroups per CU walk the work items with a grid stride,
  // so the filters are loaded once per workgroup rather than once per item.
  const int64_t max_grid = (int64_t)VGGT3_CONV_WG_PER_CU * 256;
  const unsigned n_blocks = (unsigned)(n_work < max_grid ? n_work : max_grid);
  if (bf16 && C % 128 == 0 && lds_ring_bytes<128, 2>(grid_w) <= LDS_MAX_BYTES &&
      launch_lds<128, 2, 512>(V, Vp, w, n_views, grid_h, grid_w, n_special, C, 2, stream))
    return hipGetLastError();
  if (bf16 && C % 64 == 0 && lds_ring_bytes<64, 3>(grid_w) <= LDS_MAX_BYTES &&
      launch_lds<64, 3, 256>(V, Vp, w, n_views, grid_h, grid_w, n_special, C, 3, stream))
    return hipGetLastError();
  if (bf16)
    hipLaunchKernelGGL(shortconv_kernel<true>, dim3(n_blocks), dim3(256), 0, stream, static_cast<const char*>(V),
                       static_cast<char*>(Vp), w, n_work, grid_h, grid_w, n_special, C, n_seg, n_cblk);
  else
    hipLaunchKernelGGL(shortconv_kernel<false>, dim3(n_blocks), dim3(256), 0, stream, static_cast<const char*>(V),
                       static_cast<char*>(Vp), w, n_work, grid_h, grid_w, n_special, C, n_seg, n_cblk);
  return hipGetLastError();
}

int shortconv_max_grid_w() { return MAX_W; }

}  // namespace vggt3

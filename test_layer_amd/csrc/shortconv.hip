// ShortConv2D on the value tokens: depthwise 3x3 over each view's patch grid.
//
// Paper-graph summary "VGG-T3: Offline Feed-Forward 3D Reconstruction at Scale",
// section 3.4 "Non-Linear Spatial Mixing via ShortConv2D": the value tokens of a
// view are put back on their (H/p, W/p) patch grid, mixed by one 3x3 conv and
// flattened again; per its Appendix A note, camera and register tokens bypass
// the conv. The conv is depthwise (one 3x3 filter per channel), zero padded.
//
// Design (HBM-bound stencil). One thread owns one (view, column x, segment of
// SEG rows, 4-channel group). It issues the loads of all SEG+2 input rows of
// its segment at columns x-1, x, x+1 at once (8 bytes each; about 18 KB in
// flight per wave, which is what keeps HBM busy), then computes the SEG output
// rows with a rotating 3x3 window of fp32 vectors in registers. The code is
// straight-line: rows outside the grid load as zero and only the stores of
// rows past the segment are skipped. Lanes of a wave cover consecutive channel
// groups of one token (512 contiguous bytes per wave access); the x-1 / x+1
// re-reads of neighbouring columns hit L1/L2, and workgroups are remapped so
// that each XCD walks a contiguous range of columns.
//
// Bit-exact contract: acc = +0; taps with the row offset outermost and the
// column offset innermost; acc = fl(acc + fl(w*v)), never fused (this file is
// compiled with -ffp-contract=off and the pragma below); out-of-grid taps see
// v = 0, which leaves acc unchanged; the result is rounded to bf16 with ties
// to even.
#include "common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace vggt3 {

namespace {

constexpr int SEG = 10;     // output rows per thread (37 rows -> 4 segments)
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

// One output row: acc = sum over taps, row offset outermost, column innermost.
__device__ __forceinline__ void conv_row(const float (&wt)[9][4], const float (&up)[3][4],
                                         const float (&mid)[3][4], const float (&dn)[3][4], float (&acc)[4]) {
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) acc[ch] = 0.0f;
#pragma unroll
  for (int b = 0; b < 3; ++b)
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) acc[ch] = acc[ch] + wt[b][ch] * up[b][ch];
#pragma unroll
  for (int b = 0; b < 3; ++b)
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) acc[ch] = acc[ch] + wt[3 + b][ch] * mid[b][ch];
#pragma unroll
  for (int b = 0; b < 3; ++b)
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) acc[ch] = acc[ch] + wt[6 + b][ch] * dn[b][ch];
}

template <bool BF16>
__global__ __launch_bounds__(256) void shortconv_kernel(const char* __restrict__ V, char* __restrict__ Vp,
                                                         const float* __restrict__ w, int64_t n_items,
                                                         int grid_h, int grid_w, int n_special, int C,
                                                         int n_seg, int64_t n_blocks) {
  using Tr = ConvTraits<BF16>;
  typedef typename Tr::vec_t vec_t;
  constexpr int VB = (int)sizeof(vec_t);  // bytes per 4-channel group
  const int64_t blk = xcd_remap(blockIdx.x, n_blocks);
  const int64_t item = blk * 256 + threadIdx.x;
  if (item >= n_items) return;
  // item -> (view, column x, segment, channel group); channel group fastest.
  const int CG = C / 4;
  const int cg = (int)(item % CG);
  int64_t rest = item / CG;
  const int seg = (int)(rest % n_seg);
  rest /= n_seg;
  const int x = (int)(rest % grid_w);
  const int64_t view = rest / grid_w;
  const int64_t row_bytes = (int64_t)C * Tr::ESZ;
  const int64_t tpv = (int64_t)n_special + (int64_t)grid_h * grid_w;
  const char* vview = V + view * tpv * row_bytes + (int64_t)cg * VB;
  char* oview = Vp + view * tpv * row_bytes + (int64_t)cg * VB;

  if (x == 0 && seg == 0) {
    for (int s = 0; s < n_special; ++s)
      *reinterpret_cast<vec_t*>(oview + s * row_bytes) = *reinterpret_cast<const vec_t*>(vview + s * row_bytes);
  }

  const int y0 = seg * SEG;
  const int64_t grid_row = (int64_t)grid_w * row_bytes;  // bytes from one grid row to the next
  const char* src = vview + (int64_t)n_special * row_bytes + (int64_t)x * row_bytes;  // (y = 0, x)
  char* dst = oview + (int64_t)n_special * row_bytes + (int64_t)x * row_bytes;
  const bool has_l = x > 0, has_r = x + 1 < grid_w;

  // Loads of input rows y0-1 .. y0+SEG at columns x-1, x, x+1. Every load is
  // issued (from a clamped, in-grid address) and taps outside the grid are
  // then replaced by zero with a select: with no conditional loads the
  // compiler's load-counter waits stay exact, so all 36 loads stay in flight.
  const int xl = has_l ? -1 : 0, xr = has_r ? 1 : 0;
  vec_t raw[SEG + 2][3];
#pragma unroll
  for (int k = 0; k < SEG + 2; ++k) {
    const int y = y0 - 1 + k;
    const int yc = y < 0 ? 0 : (y >= grid_h ? grid_h - 1 : y);
    const char* p = src + (int64_t)yc * grid_row;
    raw[k][0] = *reinterpret_cast<const vec_t*>(p + xl * row_bytes);
    raw[k][1] = *reinterpret_cast<const vec_t*>(p);
    raw[k][2] = *reinterpret_cast<const vec_t*>(p + xr * row_bytes);
  }
#pragma unroll
  for (int k = 0; k < SEG + 2; ++k) {
    const int y = y0 - 1 + k;
    const bool in = y >= 0 && y < grid_h;
    if (!(in && has_l)) raw[k][0] = vec_t{};
    if (!in) raw[k][1] = vec_t{};
    if (!(in && has_r)) raw[k][2] = vec_t{};
  }

  float wt[9][4];
#pragma unroll
  for (int ch = 0; ch < 4; ++ch)
#pragma unroll
    for (int t = 0; t < 9; ++t) wt[t][ch] = w[(int64_t)(cg * 4 + ch) * 9 + t];

  float rA[3][4], rB[3][4], rC[3][4], acc[4];
  auto widen_row = [&](int k, float (&row)[3][4]) {
#pragma unroll
    for (int b = 0; b < 3; ++b) Tr::widen(raw[k][b], row[b]);
  };
  auto store_row = [&](int k) {
    const int y = y0 + k;
    if (y < grid_h) *reinterpret_cast<vec_t*>(dst + (int64_t)y * grid_row) = Tr::narrow(acc);
  };
  widen_row(0, rA);
  widen_row(1, rB);
#pragma unroll
  for (int k = 0; k < SEG; k += 3) {
    widen_row(k + 2, rC);
    conv_row(wt, rA, rB, rC, acc);
    store_row(k);
    if (k + 1 < SEG) {
      widen_row(k + 3, rA);
      conv_row(wt, rB, rC, rA, acc);
      store_row(k + 1);
    }
    if (k + 2 < SEG) {
      widen_row(k + 4, rB);
      conv_row(wt, rC, rA, rB, acc);
      store_row(k + 2);
    }
  }
}

}  // namespace

hipError_t launch_shortconv(const void* V, void* Vp, const float* w, int64_t n_views, int grid_h,
                            int grid_w, int n_special, int C, bool bf16, hipStream_t stream) {
  const int n_seg = (grid_h + SEG - 1) / SEG;
  const int64_t n_items = n_views * grid_w * (int64_t)n_seg * (C / 4);
  if (n_items == 0) return hipSuccess;
  const int64_t n_blocks = (n_items + 255) / 256;
  if (bf16)
    hipLaunchKernelGGL(shortconv_kernel<true>, dim3((unsigned)n_blocks), dim3(256), 0, stream,
                       static_cast<const char*>(V), static_cast<char*>(Vp), w, n_items, grid_h, grid_w,
                       n_special, C, n_seg, n_blocks);
  else
    hipLaunchKernelGGL(shortconv_kernel<false>, dim3((unsigned)n_blocks), dim3(256), 0, stream,
                       static_cast<const char*>(V), static_cast<char*>(Vp), w, n_items, grid_h, grid_w,
                       n_special, C, n_seg, n_blocks);
  return hipGetLastError();
}

int shortconv_max_grid_w() { return MAX_W; }

}  // namespace vggt3

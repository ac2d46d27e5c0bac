// ShortConv2D on the value tokens: depthwise 3x3 over each view's patch grid.
//
// Paper-graph summary "VGG-T3: Offline Feed-Forward 3D Reconstruction at Scale",
// section 3.4 "Non-Linear Spatial Mixing via ShortConv2D": the value tokens of a
// view are put back on their (H/p, W/p) patch grid, mixed by one 3x3 conv and
// flattened again; per its Appendix A note, camera and register tokens bypass
// the conv. The conv is depthwise (one 3x3 filter per channel), zero padded.
//
// Design (HBM-bound stencil): one thread owns one (view, column x, 16-byte
// channel group) and walks down the column keeping a 3x3 window of fp32
// vectors in registers, so each input row is loaded once per thread and the
// x-1 / x+1 loads of neighbouring threads hit L1/L2. Lanes of a wave cover
// consecutive channel groups of one token, so every load and store is a
// contiguous 1 KB wave transaction. Workgroups are remapped so that each XCD
// walks a contiguous range of columns (the x+-1 re-reads stay in its L2).
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

template <bool BF16>
struct ConvTraits;
template <>
struct ConvTraits<true> {
  static constexpr int VEC = 8;  // 8 bf16 = 16 bytes
  __device__ static void load(const void* base, int64_t elem, float (&v)[8]) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(q[i]);
      v[2 * i + 1] = bf16_hi(q[i]);
    }
  }
  __device__ static void store(void* base, int64_t elem, const float (&v)[8]) {
    u32x4 q;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(base) + elem) = q;
  }
  __device__ static void copy(const void* src, void* dst, int64_t elem) {
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(dst) + elem) =
        *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(src) + elem);
  }
};
template <>
struct ConvTraits<false> {
  static constexpr int VEC = 4;  // 4 fp32 = 16 bytes
  __device__ static void load(const void* base, int64_t elem, float (&v)[4]) {
    const f32x4 q = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = q[i];
  }
  __device__ static void store(void* base, int64_t elem, const float (&v)[4]) {
    f32x4 q;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = v[i];
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + elem) = q;
  }
  __device__ static void copy(const void* src, void* dst, int64_t elem) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dst) + elem) =
        *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(src) + elem);
  }
};

template <bool BF16>
__global__ __launch_bounds__(256) void shortconv_kernel(const void* __restrict__ V, void* __restrict__ Vp,
                                                         const float* __restrict__ w, int64_t n_items,
                                                         int grid_h, int grid_w, int n_special, int C,
                                                         int64_t n_blocks) {
  using Tr = ConvTraits<BF16>;
  constexpr int VEC = Tr::VEC;
  const int64_t blk = xcd_remap(blockIdx.x, n_blocks);
  const int64_t item = blk * 256 + threadIdx.x;
  if (item >= n_items) return;
  const int CG = C / VEC;
  const int cg = (int)(item % CG);
  const int64_t vx = item / CG;
  const int x = (int)(vx % grid_w);
  const int64_t view = vx / grid_w;
  const int c0 = cg * VEC;
  const int64_t tpv = (int64_t)n_special + (int64_t)grid_h * grid_w;
  const int64_t view_base = view * tpv;  // first token of the view

  if (x == 0) {
    for (int s = 0; s < n_special; ++s) Tr::copy(V, Vp, (view_base + s) * C + c0);
  }

  // Filter taps for this thread's channels: wt[tap][ch], tap = (a+1)*3 + (b+1).
  float wt[9][VEC];
#pragma unroll
  for (int ch = 0; ch < VEC; ++ch) {
#pragma unroll
    for (int t = 0; t < 9; ++t) wt[t][ch] = w[(int64_t)(c0 + ch) * 9 + t];
  }

  const int64_t patch_base = view_base + n_special;
  // Window rows: win[0] = row y-1, win[1] = row y, win[2] = row y+1; columns x-1, x, x+1.
  float win[3][3][VEC];
#pragma unroll
  for (int b = 0; b < 3; ++b)
#pragma unroll
    for (int ch = 0; ch < VEC; ++ch) win[0][b][ch] = 0.0f;

  auto load_row = [&](int y, float (&row)[3][VEC]) {
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const int xx = x + b - 1;
      if (y < grid_h && xx >= 0 && xx < grid_w) {
        Tr::load(V, (patch_base + (int64_t)y * grid_w + xx) * C + c0, row[b]);
      } else {
#pragma unroll
        for (int ch = 0; ch < VEC; ++ch) row[b][ch] = 0.0f;
      }
    }
  };

  load_row(0, win[1]);
  for (int y = 0; y < grid_h; ++y) {
    load_row(y + 1, win[2]);
    float acc[VEC];
#pragma unroll
    for (int ch = 0; ch < VEC; ++ch) acc[ch] = 0.0f;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
#pragma unroll
      for (int b = 0; b < 3; ++b) {
#pragma unroll
        for (int ch = 0; ch < VEC; ++ch) {
          const float p = wt[a * 3 + b][ch] * win[a][b][ch];
          acc[ch] = acc[ch] + p;
        }
      }
    }
    Tr::store(Vp, (patch_base + (int64_t)y * grid_w + x) * C + c0, acc);
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
      for (int ch = 0; ch < VEC; ++ch) {
        win[0][b][ch] = win[1][b][ch];
        win[1][b][ch] = win[2][b][ch];
      }
  }
}

hipError_t launch_shortconv(const void* V, void* Vp, const float* w, int64_t n_views, int grid_h,
                            int grid_w, int n_special, int C, bool bf16, hipStream_t stream) {
  const int VEC = bf16 ? 8 : 4;
  const int64_t n_items = n_views * grid_w * (int64_t)(C / VEC);
  if (n_items == 0) return hipSuccess;
  const int64_t n_blocks = (n_items + 255) / 256;
  if (bf16)
    hipLaunchKernelGGL(shortconv_kernel<true>, dim3((unsigned)n_blocks), dim3(256), 0, stream, V, Vp, w,
                       n_items, grid_h, grid_w, n_special, C, n_blocks);
  else
    hipLaunchKernelGGL(shortconv_kernel<false>, dim3((unsigned)n_blocks), dim3(256), 0, stream, V, Vp, w,
                       n_items, grid_h, grid_w, n_special, C, n_blocks);
  return hipGetLastError();
}

}  // namespace vggt3

// Internal launchers of the TTT-layer kernels (host side) and launch helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vggt3 {

// The dispatcher hands workgroup b to XCD b % 8 (8 XCDs, each with its own L2).
// Remap so that each XCD processes a contiguous range of logical workgroups:
// neighbouring tiles (which share halo rows or weights) then share one L2.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t n) {
  const int64_t q = n / kNumXcd, r = n % kNumXcd;
  const int64_t xcd = b % kNumXcd, idx = b / kNumXcd;
  return xcd * q + (xcd < r ? xcd : r) + idx;
}

// Chunking of the Eq. 5 gradient split: the tokens are cut into P chunks
// (P a power of two, a function of n_tokens and n_heads only, never of the
// device), one workgroup per (head, chunk); partial gradients are summed by a
// fixed pairwise tree, so results do not depend on the GPU's CU count.
constexpr int kMaxChunks = 64;
int ttt_num_chunks(int64_t n_tokens, int n_heads, int tile_tokens);
// Tokens per tile of the gradient kernels: the unit a chunk is cut in. The
// kernels assert that they tile by these, and the chunk count is taken from them.
constexpr int kGradTileBf16 = 32;
constexpr int kGradTileF32 = 16;

// Widest patch-grid row the ShortConv2D kernel stages in LDS.
int shortconv_max_grid_w();
hipError_t launch_shortconv(const void* V, void* Vp, const float* w, int64_t n_views, int grid_h,
                            int grid_w, int n_special, int C, bool bf16, hipStream_t stream);
// Filter size ksize (3: the kernel above; 5: the k x k variant kernel).
hipError_t launch_shortconv_k(const void* V, void* Vp, const float* w, int64_t n_views, int grid_h, int grid_w,
                              int n_special, int C, int ksize, bool bf16, hipStream_t stream);

// Patch-grid geometry for the ShortConv2D fused into the gradient pass: each
// view is n_special tokens, then grid_h x grid_w patch tokens row by row
// (tpv tokens in all). magic_* = ceil(2^32 / divisor), 0 for a divisor of 1,
// so that v_mul_hi divides any value below 2^16 exactly.
struct ConvGeom {
  int tpv, n_special, grid_h, grid_w;
  uint32_t magic_tpv, magic_gw;
};

// Per-(head, chunk) fp32 gradient and loss partials.
// part: [n_heads][P][3*d*m], loss_part: [n_heads][P]. dot selects the
// dot-product loss -sum T(k).v' instead of sum (1/d)||T(k) - v'||^2.
// With loss false the loss partials are written as NaN and the loss work is skipped.
hipError_t launch_grad_partial_bf16(const void* K, const void* Vp, const float* theta, float* part,
                                    float* loss_part, int64_t n_tokens, int n_heads, int P, bool dot, bool loss,
                                    hipStream_t stream);
// The same partials with V' = ShortConv2D(V) formed inside the pass (bf16,
// d = 64, m = 128, 3x3 filters conv_w [C][3][3] fp32, grid_w at most
// conv_fused_max_grid_w(), n_tokens a whole number of views, tpv + 31 < 2^16).
// Vp_out, if not NULL, receives V' (bf16, like K).
int conv_fused_max_grid_w();
hipError_t launch_grad_partial_conv_bf16(const void* K, const void* V, const float* conv_w, void* Vp_out,
                                         const ConvGeom& geo, const float* theta, float* part, float* loss_part,
                                         int64_t n_tokens, int n_heads, int P, bool dot, bool loss,
                                         hipStream_t stream);
// fp32 arithmetic; bf16_tokens: K and V' are bf16 (only at d = 16, m = 32).
hipError_t launch_grad_partial_f32(const void* K, const void* Vp, const float* theta, float* part,
                                   float* loss_part, int64_t n_tokens, int n_heads, int d, int m, int P,
                                   bool dot, bool bf16_tokens, hipStream_t stream);

// Muon update theta -= lr * NS(grad) for every per-head weight matrix, NS the
// `ns_steps`-step quintic Newton-Schulz orthogonalisation (fp32).
hipError_t launch_muon_apply(float* theta, const float* grad, float lr, int n_heads, int d, int m, int ns_steps,
                             hipStream_t stream);

// Fixed-tree reduction of the partials, then (mode) either
//   kApply:   theta -= lr * g            (write step), loss_out[h] = loss
//   kStore:   grad = g,  loss_out = loss
//   kAccum:   grad += g, loss_out += loss
enum ReduceMode { kApply = 0, kStore = 1, kAccum = 2 };
hipError_t launch_reduce(const float* part, const float* loss_part, int n_heads, int P, int per_head,
                         ReduceMode mode, float* theta_or_grad, float lr, float* loss_out,
                         hipStream_t stream);
hipError_t launch_apply(float* theta, const float* grad, float lr, int64_t count, hipStream_t stream);
hipError_t launch_fill(float* dst, float value, int64_t count, hipStream_t stream);

hipError_t launch_read_bf16(const void* Q, const float* theta, void* O, int64_t n_tokens, int n_heads,
                            hipStream_t stream);
hipError_t launch_read_f32(const void* Q, const float* theta, void* O, int64_t n_tokens, int n_heads,
                           int d, int m, bool bf16_tokens, hipStream_t stream);

}  // namespace vggt3

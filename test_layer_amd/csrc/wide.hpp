// Host-side interface of the wide-MLP kernels (one 1024 -> 4096 -> 1024
// SwiGLU over the whole token width).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vggt3 {
namespace wide {

constexpr int kD = 1024;          // inputs / outputs
constexpr int kM = 4096;          // hidden units
constexpr int kTile = 256;        // GEMM tile (rows and columns)
constexpr int kSplit = 8;         // split-K slices of the token-reduction GEMMs
constexpr int64_t kChunk = 131072;  // tokens per chunk of the write and the read

// Epilogues of the GEMM kernel.
enum Epi {
  EPI_SWIGLU = 0,    // [G|U] -> H (row-major), A and GP (C-native)
  EPI_SWIGLU_H = 1,  // [G|U] -> H only (read)
  EPI_Y_LOSS = 2,    // Y -> -Y (row-major), sum (Y - V')^2 per workgroup
  EPI_Y_STORE = 3,   // Y -> O (row-major)
  EPI_DH = 4,        // D -> [D*GP | D*A] (row-major [rows][2m])
  EPI_PARTIAL = 6    // fp32 split-K partial (C-native), stored or added
};

// C[M x N] = sum over segments s < nseg of A_s B_s, each a K-deep product.
// Token-major GEMMs (all but EPI_PARTIAL): A_s(i, k) = A[s][i * lda[s] + k],
// B_s(k, j) = B[s][j * ldb[s] + k]; M may be ragged, N and K are multiples of
// the tile and of 64. EPI_PARTIAL: A_s(i, k) = A[s][k * lda[s] + i],
// B_s(k, j) = B[s][k * ldb[s] + j] (reductions over tokens k, ragged K), split
// into S slices of k. a_rows / b_rows (EPI_PARTIAL only) are the k rows each
// operand has; reads past them are clamped. Of every product one operand must
// hold zeros in rows K .. K rounded up to 64 and have those rows (the
// epilogues EPI_SWIGLU and EPI_DH write them for H and [dG | dU]).
struct GemmArgs {
  int64_t M, N, K;
  int nseg;
  int S;
  const uint16_t* A[2];
  const uint16_t* B[2];
  int64_t lda[2], ldb[2];
  int64_t a_rows[2], b_rows[2];
  uint16_t* out0;
  uint16_t* out1;
  uint16_t* out2;
  const uint16_t* in0;
  const uint16_t* in1;
  int64_t ldo, ldi;
  float* fout;
  int accumulate;
};

hipError_t launch_gemm(int epi, const GemmArgs& g, hipStream_t stream);
hipError_t launch_pack(const float* theta, uint16_t* wgu, uint16_t* wdt, uint16_t* wdn, int d, int m,
                       hipStream_t stream);
// Blocks of the partials reduction (one 256-thread block per 256 gradient
// elements); with wd_dot it writes one W_d . g partial per block.
constexpr unsigned reduce_blocks(int d, int m) { return (unsigned)((3 * (int64_t)d * m + 255) / 256); }
hipError_t launch_reduce_partials(const float* p_gu, const float* p_d, int S, int d, int m, float scale, int mode,
                                  float* dst, float lr, const float* theta, float* wd_dot, hipStream_t stream);
hipError_t launch_sum(const float* x, int64_t n, float scale, int accumulate, float* out, hipStream_t stream);

// Muon update theta -= lr * NS(grad) of the three matrices (fp32 GEMMs), with a
// scratch of muon_workspace_floats(d, m) floats.
size_t muon_workspace_floats(int d, int m);
hipError_t launch_muon(float* theta, const float* grad, float lr, int d, int m, int ns_steps, float* ws,
                       hipStream_t stream);

}  // namespace wide
}  // namespace vggt3

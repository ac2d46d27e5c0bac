// Read pass (bf16 MFMA): O = T_theta(Q) per head for d = 64, m = 128.
//
// Query step of the fast-weight MLP (paper-graph summary "VGG-T3: Offline
// Feed-Forward 3D Reconstruction at Scale", section 3.4, Eq. 4: o_i =
// T_theta(q_i); with a frozen theta* this is also the query mode for unseen
// views), T(x) = (silu(x W_g) * (x W_u)) W_d without biases.
#include "bf16_ops.hpp"
#include "kernels.hpp"

namespace vggt3 {
namespace {

constexpr int D = 64;
constexpr int M = 128;
constexpr int KP = D + 8;
constexpr int HP = M + 8;
constexpr int DM = D * M;
constexpr int PER_HEAD = 3 * DM;

// ---------------------------------------------------------------------------
// Read pass O = T(Q) per head. Tokens run across lanes here (MFMA columns),
// so the chain G^T = W_g^T Q^T -> H^T -> Y^T = W_d^T H^T contracts over e and
// then over hidden units with no transposes: each H^T tile is consumed from
// registers. Weights sit in LDS, pre-permuted to match the operand orders.
// Each wave handles 32 tokens per iteration.
// ---------------------------------------------------------------------------
constexpr int RT = 32;  // tokens per wave iteration
constexpr int NW = 8;   // waves per workgroup
// Two workgroups per CU (four waves per SIMD) need at most 128 VGPRs per lane;
// the kernel compiles to 128 (check num_vgpr in the assembly after changes).

__global__ __launch_bounds__(512, 2) void read_bf16_kernel(const uint16_t* __restrict__ Q,
                                                           const float* __restrict__ theta,
                                                           uint16_t* __restrict__ O, int64_t n_tokens,
                                                           int n_heads, int P, int64_t n_blocks) {
  __shared__ __attribute__((aligned(16))) uint16_t WgP[M * KP];
  __shared__ __attribute__((aligned(16))) uint16_t WuP[M * KP];
  __shared__ __attribute__((aligned(16))) uint16_t WdP[D * HP];

  const int64_t blk = xcd_remap(blockIdx.x, n_blocks);
  const int head = (int)(blk / P);
  const int chunk = (int)(blk % P);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so tile offsets stay scalar
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t C = (int64_t)n_heads * D;
  const float* th = theta + (int64_t)head * PER_HEAD;

  // A operand of G^T for k-step ks: lane (row hid, half hh) supplies
  // W_g[e = 32hh + 8ks + j][hid]; stored at WgP[hid][16ks + 8hh + j].
  for (int idx = tid; idx < M * D; idx += 64 * NW) {
    const int hid = idx / D, kk = idx % D;
    const int ks = kk >> 4, h2 = (kk >> 3) & 1, j = kk & 7;
    const int e = 32 * h2 + 8 * ks + j;
    WgP[hid * KP + kk] = f32_to_bf16_bits(th[e * M + hid]);
    WuP[hid * KP + kk] = f32_to_bf16_bits(th[DM + e * M + hid]);
  }
  // A operand of Y^T for k-step s: lane (row o, half hh) supplies
  // W_d[hid = 16s + 8(j/4) + 4hh + j%4][o] (the register order of H^T).
  for (int idx = tid; idx < D * M; idx += 64 * NW) {
    const int o = idx / M, kk = idx % M;
    const int s = kk >> 4, h2 = (kk >> 3) & 1, j = kk & 7;
    const int hid = 16 * s + 8 * (j >> 2) + 4 * h2 + (j & 3);
    WdP[o * HP + kk] = f32_to_bf16_bits(th[2 * DM + hid * D + o]);
  }
  __syncthreads();

  const int64_t n_tiles = (n_tokens + RT - 1) / RT;
  const int64_t tile_begin = n_tiles * chunk / P;
  const int64_t tile_end = n_tiles * (chunk + 1) / P;

  // Each wave walks tiles tile_begin + w, + NW, ...; the next tile's queries
  // are loaded while the current one computes. Q and O are accessed through
  // buffer descriptors built per tile from 64-bit scalar arithmetic, based at
  // the tile's first token and this head, with a range that ends at the
  // tensor's end: rows at or past n_tokens read as zeros and their stores are
  // dropped, so loads and stores are unconditional and the lane offsets fixed.
  const int lane_off = (l32 * (int)C + 32 * hh) * 2;
  auto tile_res = [&](const uint16_t* base, int64_t tile) {
    const int64_t t0 = tile * RT;
    const int64_t range = (n_tokens - t0) * C * 2 - (int64_t)head * D * 2;
    const int nrec = (int)(range > 0x7fffffffLL ? 0x7fffffffLL : (range > 0 ? range : 0));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + t0 * C + (int64_t)head * D), (short)0, nrec, 0x00020000);
  };
  auto load_q = [&](int64_t tile, u32x4 (&dst)[4]) {
    const __amdgpu_buffer_rsrc_t r = tile_res(Q, tile);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      dst[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off + 16 * ks, 0, 0));
  };
  // Two query register sets alternate (no loop-carried copies, so the load
  // waits stay exact): tile k computes from one set while tile k+1 loads into
  // the other.
  auto compute_tile = [&](int64_t tile, const u32x4 (&qr)[4]) {
    bf16x8 q[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) q[ks] = as_bf16x8(qr[ks]);
    // The weight reads below are loop-invariant; an opaque zero offset keeps the
    // compiler from hoisting 48 operand vectors into registers (and spilling).
    int lds0 = 0;
    asm volatile("" : "+v"(lds0));
    f32x16 accY[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x16 g = f32x16{}, u = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int off = lds0 + (32 * mt + l32) * KP + 16 * ks + 8 * hh;
        g = mfma32(ld_op(&WgP[off]), q[ks], g);
        u = mfma32(ld_op(&WuP[off]), q[ks], u);
      }
      float h[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float s = sigmoid_fast(g[r]);
        h[r] = g[r] * s * u[r];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 hop = pack8(&h[8 * half]);
        const int s = 2 * mt + half;
#pragma unroll
        for (int ot = 0; ot < 2; ++ot) {
          accY[ot] = mfma32(ld_op(&WdP[lds0 + (32 * ot + l32) * HP + 16 * s + 8 * hh]), hop, accY[ot]);
        }
      }
    }
    // Output row o of Y^T tile ot is 8q + 4hh + i (q = r/4, i = r%4) in lane
    // half hh. Exchanging the q-odd quads of the low half with the q-even
    // quads of the high half (v_permlane32_swap) gives every lane 8
    // consecutive outputs, stored as one 16-byte write.
    const __amdgpu_buffer_rsrc_t ores = tile_res(O, tile);
#pragma unroll
    for (int ot = 0; ot < 2; ++ot) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const f32x16& a = accY[ot];
        const uint32_t y0 = pack_bf16x2(a[8 * p + 0], a[8 * p + 1]), y1 = pack_bf16x2(a[8 * p + 2], a[8 * p + 3]);
        const uint32_t x0 = pack_bf16x2(a[8 * p + 4], a[8 * p + 5]), x1 = pack_bf16x2(a[8 * p + 6], a[8 * p + 7]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(y0, x0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(y1, x1, false, false);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{s0[0], s1[0], s0[1], s1[1]}, ores,
                                               (l32 * (int)C + 32 * ot + 16 * p + 8 * hh) * 2, 0, 0);
      }
    }
  };
  u32x4 qa[4], qb[4];
  load_q(tile_begin + w, qa);
  for (int64_t tile = tile_begin + w; tile < tile_end; tile += 2 * NW) {
    load_q(tile + NW, qb);
    compute_tile(tile, qa);
    load_q(tile + 2 * NW, qa);
    if (tile + NW < tile_end) compute_tile(tile + NW, qb);
  }
}

}  // namespace

hipError_t launch_read_bf16(const void* Q, const float* theta, void* O, int64_t n_tokens, int n_heads,
                            hipStream_t stream) {
  // Enough workgroups to fill 256 CUs twice over; each handles a contiguous
  // run of 32-token tiles of one head.
  const int64_t n_tiles = (n_tokens + RT - 1) / RT;
  int64_t P = (512 + n_heads - 1) / n_heads;
  if (P > n_tiles) P = n_tiles;
  if (P < 1) P = 1;
  const int64_t n_blocks = (int64_t)n_heads * P;
  hipLaunchKernelGGL(read_bf16_kernel, dim3((unsigned)n_blocks), dim3(64 * NW), 0, stream,
                     static_cast<const uint16_t*>(Q), theta, static_cast<uint16_t*>(O), n_tokens, n_heads,
                     (int)P, n_blocks);
  return hipGetLastError();
}

}  // namespace vggt3

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
//
// All products use 16x16x32 MFMA tiles. A wave takes 32 tokens per iteration
// as two 16-token halves that share every weight operand read from LDS (one
// read feeds two MFMAs). With 16 tokens per MFMA column block, each query
// load instruction covers 16 token rows x 64 contiguous bytes and each output
// store 16 rows x 64 bytes, where 32x32 tiles touch 32 rows x 32 bytes: half
// the cache lines per memory instruction.
// ---------------------------------------------------------------------------
constexpr int RT = 32;  // tokens per wave iteration (two 16-token halves)
constexpr int NW = 8;   // waves per workgroup
// Two workgroups per CU (four waves per SIMD) need at most 128 VGPRs per lane;
// the kernel compiles to 114 without spills (check the resource usage after
// changes).

// 16x16x32 bf16 MFMA, fp32 accumulate.
//   A operand: lane l holds A[row = l%16][k = 8*(l/16) + j], j = 0..7
//   B operand: lane l holds B[k = 8*(l/16) + j][col = l%16]
//   C/D:       lane l, register r holds C[row = 4*(l/16) + r][col = l%16]
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(512, 4) void read_bf16_kernel(const uint16_t* __restrict__ Q,
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
  const int l16 = lane & 15;
  const int g = lane >> 4;  // k-quarter of an operand, row quad of a result
  const int64_t C = (int64_t)n_heads * D;
  const float* th = theta + (int64_t)head * PER_HEAD;

  // A operand of G'^T (rows hid, k = e): WgP[hid][e] = -log2(e) W_g[e][hid],
  // WuP[hid][e] = -ln(2) W_u[e][hid]. The two scales fold the exp2 argument
  // of the sigmoid into the weights: with G' = -log2(e) G and U' = -ln(2) U,
  // silu(G) U = G' U' / (1 + 2^G'), since log2(e) ln(2) = 1. That saves one
  // multiply per hidden unit; each weight is still rounded once to bf16 (after
  // its scaling). The 144-byte row pitch keeps 16 lanes reading 16 rows
  // conflict-free.
  for (int idx = tid; idx < M * D; idx += 64 * NW) {
    const int e = idx / M, hid = idx % M;
    WgP[hid * KP + e] = f32_to_bf16_bits(th[e * M + hid] * -1.4426950408889634f);
    WuP[hid * KP + e] = f32_to_bf16_bits(th[DM + e * M + hid] * -0.6931471805599453f);
  }
  // A operand of Y^T for k-step s (32 hidden units): lane (row o, quarter g)
  // supplies W_d[hid][o] for hid = 32s + 4g + j (j < 4) and 32s + 16 + 4g +
  // j - 4 (j >= 4): the order in which a lane holds H^T (rows 4g..4g+3 of the
  // two 16-row G^T tiles of that k-step).
  for (int idx = tid; idx < D * M; idx += 64 * NW) {
    const int o = idx / M, kk = idx % M;
    const int s = kk >> 5, gg = (kk >> 3) & 3, j = kk & 7;
    const int hid = 32 * s + (j < 4 ? 4 * gg + j : 16 + 4 * gg + j - 4);
    WdP[o * HP + kk] = f32_to_bf16_bits(th[2 * DM + hid * D + o]);
  }
  __syncthreads();

  const int64_t n_tiles = (n_tokens + RT - 1) / RT;
  const int64_t tile_begin = n_tiles * chunk / P;
  const int64_t tile_end = n_tiles * (chunk + 1) / P;

  // Q and O are accessed through buffer descriptors built per tile from
  // 64-bit scalar arithmetic, based at the tile's first token and this head,
  // with a range that ends at the tensor's end: rows at or past n_tokens read
  // as zeros and their stores are dropped, so loads and stores are
  // unconditional and the lane offsets fixed. Lane (token l16, quarter g)
  // loads channels 32ks + 8g .. +7 of its token for k-step ks.
  const int lane_off = (l16 * (int)C + 8 * g) * 2;
  auto tile_res = [&](const uint16_t* base, int64_t tile) {
    const int64_t t0 = tile * RT;
    const int64_t range = (n_tokens - t0) * C * 2 - (int64_t)head * D * 2;
    const int nrec = (int)(range > 0x7fffffffLL ? 0x7fffffffLL : (range > 0 ? range : 0));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + t0 * C + (int64_t)head * D), (short)0, nrec, 0x00020000);
  };
  auto compute_tile = [&](int64_t tile) {
    const __amdgpu_buffer_rsrc_t qres = tile_res(Q, tile);
    bf16x8 q[2][2];  // [half b][k-step ks]
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        q[b][ks] = as_bf16x8(__builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(qres, lane_off + 32 * (int)C * b + 64 * ks, 0, 0)));
    // The weight reads below are loop-invariant; an opaque zero offset keeps the
    // compiler from hoisting the operand vectors into registers (and spilling).
    int lds0 = 0;
    asm volatile("" : "+v"(lds0));
    f32x4 accY[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int ot = 0; ot < 4; ++ot) accY[b][ot] = f32x4{};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // G'^T and U'^T rows 32s..32s+15 (tile 0) and 32s+16..32s+31 (tile 1).
      f32x4 g0[2], g1[2], u0[2], u1[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) g0[b] = g1[b] = u0[b] = u1[b] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int off0 = lds0 + (32 * s + l16) * KP + 32 * ks + 8 * g;
        const int off1 = off0 + 16 * KP;
        const bf16x8 ag0 = ld_op(&WgP[off0]), au0 = ld_op(&WuP[off0]);
        const bf16x8 ag1 = ld_op(&WgP[off1]), au1 = ld_op(&WuP[off1]);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          g0[b] = mfma16(ag0, q[b][ks], g0[b]);
          u0[b] = mfma16(au0, q[b][ks], u0[b]);
          g1[b] = mfma16(ag1, q[b][ks], g1[b]);
          u1[b] = mfma16(au1, q[b][ks], u1[b]);
        }
      }
      // H^T = silu(G^T) * U^T = G'^T U'^T / (1 + 2^G'^T), packed as the B
      // operand of k-step s.
      bf16x8 hop[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float h[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          h[r] = g0[b][r] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g0[b][r])) * u0[b][r];
          h[4 + r] = g1[b][r] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g1[b][r])) * u1[b][r];
        }
        hop[b] = pack8(h);
      }
#pragma unroll
      for (int ot = 0; ot < 4; ++ot) {
        const bf16x8 wd = ld_op(&WdP[lds0 + (16 * ot + l16) * HP + 32 * s + 8 * g]);
#pragma unroll
        for (int b = 0; b < 2; ++b) accY[b][ot] = mfma16(wd, hop[b], accY[b][ot]);
      }
    }
    // Lane (token l16, quad g) holds outputs 16ot + 4g .. +3 of Y^T tile ot.
    // v_permlane16_swap exchanges the odd row groups of tile 2p with the even
    // row groups of tile 2p+1, after which quad g holds the 8 consecutive
    // outputs 32p + 16(g&1) + 8(g>>1) .. +7, stored as one 16-byte write.
    const __amdgpu_buffer_rsrc_t ores = tile_res(O, tile);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const f32x4& x = accY[b][2 * p];
        const f32x4& y = accY[b][2 * p + 1];
        const uint32_t xa = pack_bf16x2(x[0], x[1]), xb = pack_bf16x2(x[2], x[3]);
        const uint32_t ya = pack_bf16x2(y[0], y[1]), yb = pack_bf16x2(y[2], y[3]);
        const auto sa = __builtin_amdgcn_permlane16_swap(xa, ya, false, false);
        const auto sb = __builtin_amdgcn_permlane16_swap(xb, yb, false, false);
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{sa[0], sb[0], sa[1], sb[1]}, ores,
            ((16 * b + l16) * (int)C + 32 * p + 16 * (g & 1) + 8 * (g >> 1)) * 2, 0, 0);
      }
  };
  // Each wave walks tiles tile_begin + w, + NW, ... and loads a tile's
  // queries just before computing it: the other waves on the SIMD cover the
  // load latency, and no second query register set is held.
  for (int64_t tile = tile_begin + w; tile < tile_end; tile += NW) compute_tile(tile);
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

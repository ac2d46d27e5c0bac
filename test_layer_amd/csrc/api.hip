// C ABI of the TTT layer: argument validation and launch sequencing.
// Every check runs on the host before anything is enqueued.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/vggt3.h"
#include "kernels.hpp"
#include "wide.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return VGGT3_OK;
}

int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(VGGT3_EHIP, "%s: %s", what, hipGetErrorString(e));
  return VGGT3_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  if (a == nullptr || b == nullptr || an == 0 || bn == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

bool valid_dtype(int32_t dt) { return dt == VGGT3_BF16 || dt == VGGT3_F32; }
size_t elem_size(int32_t dt) { return dt == VGGT3_BF16 ? 2 : 4; }

// The pages' full-width MLP: one 1024 -> 4096 -> 1024 SwiGLU (one "head").
bool is_wide(int32_t d, int32_t m) { return d == vggt3::wide::kD && m == vggt3::wide::kM; }

// Shapes the library has kernels for.
bool supported_mlp(int32_t dt, int32_t d, int32_t m) {
  if (dt == VGGT3_BF16) return (d == 64 && m == 128) || (d == 16 && m == 32) || is_wide(d, m);
  if (dt == VGGT3_F32) return (d == 16 && m == 32) || (d == 64 && m == 128);
  return false;
}

// The fp32 vector kernels serve the fp32 mode and, with bf16 token tensors,
// the bf16 (16, 32) shape (too narrow for the 32-wide MFMA tiles).
bool f32_kernels(int32_t dt, int32_t d, int32_t m) { return dt == VGGT3_F32 || (d == 16 && m == 32); }

// Token tile of the gradient kernel that serves (dtype, d, m): the unit of the
// Eq. 5 chunking.
int tile_tokens(int32_t dt, int32_t d, int32_t m) {
  return f32_kernels(dt, d, m) ? vggt3::kGradTileF32 : vggt3::kGradTileBf16;
}

hipError_t launch_read_any(const void* Q, const float* theta, void* O, int64_t n, int32_t H, int32_t d, int32_t m,
                           int32_t dt, hipStream_t s) {
  return f32_kernels(dt, d, m) ? vggt3::launch_read_f32(Q, theta, O, n, H, d, m, dt == VGGT3_BF16, s)
                               : vggt3::launch_read_bf16(Q, theta, O, n, H, s);
}

struct MlpArgs {
  int64_t n;
  int32_t H, d, m, dt;
};

int check_mlp(const MlpArgs& a) {
  if (!valid_dtype(a.dt)) return fail(VGGT3_EINVAL, "dtype %d is not VGGT3_BF16 or VGGT3_F32", a.dt);
  if (a.n < 0) return fail(VGGT3_EINVAL, "n_tokens = %lld < 0", (long long)a.n);
  if (a.H < 1 || a.d < 1 || a.m < 1)
    return fail(VGGT3_EINVAL, "n_heads/d_head/d_hidden must be >= 1 (got %d/%d/%d)", a.H, a.d, a.m);
  if (!supported_mlp(a.dt, a.d, a.m))
    return fail(VGGT3_EUNSUPPORTED, "no %s kernel for d_head = %d, d_hidden = %d",
                a.dt == VGGT3_BF16 ? "bf16" : "f32", a.d, a.m);
  if ((int64_t)a.H * a.d > (int64_t)1 << 20) return fail(VGGT3_EUNSUPPORTED, "too many channels");
  if (is_wide(a.d, a.m) && a.H != 1)
    return fail(VGGT3_EUNSUPPORTED, "the %d -> %d -> %d MLP takes n_heads = 1 (got %d)", a.d, a.m, a.d, a.H);
  return VGGT3_OK;
}

size_t theta_bytes(const MlpArgs& a) { return (size_t)a.H * 3 * a.d * a.m * sizeof(float); }
size_t token_bytes(const MlpArgs& a) { return (size_t)a.n * a.H * a.d * elem_size(a.dt); }

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Workspace: [per-chunk gradient partials | per-chunk loss partials | one
// reduced gradient (the Muon step's input)], each 256-byte aligned.
struct WsLayout {
  size_t part, loss, grad, total;
};
WsLayout ws_layout(const MlpArgs& a, int P) {
  WsLayout l;
  l.part = 0;
  l.loss = round256((size_t)a.H * P * 3 * a.d * a.m * sizeof(float));
  l.grad = l.loss + round256((size_t)a.H * P * sizeof(float));
  l.total = l.grad + round256((size_t)a.H * 3 * a.d * a.m * sizeof(float));
  return l;
}

// Workspace of the wide MLP (write and read), for tokens processed in chunks
// of at most wide::kChunk: bf16 GEMM operands of theta, the chunk's
// intermediates, the split-K gradient partials, one reduced gradient, one
// chunk's loss partials and the Newton-Schulz scratch of the Muon update.
struct WideWs {
  int64_t ct, ctp, nchunks, loss_stride;
  size_t wgu, wdt, wdn, h, a, gp, dgu, y, pgu, pd, grad, loss, ns, total, read_total;
};
WideWs wide_ws(int64_t n) {
  namespace w = vggt3::wide;
  WideWs l{};
  l.ct = n < w::kChunk ? n : w::kChunk;
  if (l.ct < 1) l.ct = 1;
  l.ctp = (l.ct + w::kTile - 1) / w::kTile * w::kTile;
  l.nchunks = (n + l.ct - 1) / l.ct;
  l.loss_stride = (l.ctp / w::kTile) * (w::kM / w::kTile);
  const size_t d = w::kD, m = w::kM, ctp = (size_t)l.ctp;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round256(bytes);
    return at;
  };
  l.wgu = take(2 * m * d * 2);
  l.wdt = take(d * m * 2);
  l.wdn = take(m * d * 2);
  l.h = take(ctp * m * 2);
  l.read_total = o;
  l.a = take(ctp * m * 2);
  l.gp = take(ctp * m * 2);
  l.dgu = take(ctp * 2 * m * 2);
  l.y = take(ctp * d * 2);
  l.pgu = take((size_t)w::kSplit * d * 2 * m * 4);
  l.pd = take((size_t)w::kSplit * m * d * 4);
  l.grad = take(3 * d * m * 4);
  l.loss = take((size_t)(l.loss_stride > (int64_t)w::reduce_blocks(w::kD, w::kM) ? l.loss_stride
                                                                                  : w::reduce_blocks(w::kD, w::kM)) * 4);
  l.ns = take(w::muon_workspace_floats(w::kD, w::kM) * 4);
  l.total = o;
  return l;
}

size_t workspace_bytes(const MlpArgs& a, int* P_out) {
  if (is_wide(a.d, a.m)) {
    if (P_out) *P_out = 1;
    return a.n == 0 ? 0 : wide_ws(a.n).total;
  }
  const int P = vggt3::ttt_num_chunks(a.n, a.H, tile_tokens(a.dt, a.d, a.m));
  if (P_out) *P_out = P;
  if (a.n == 0) return 0;
  return ws_layout(a, P).total;
}

// One gradient pass of the wide MLP over all n tokens at theta: the gradient
// (times `scale` inside the reduce) goes to dst in `mode` (apply with lr,
// store, accumulate); the loss to loss_out (stored, or added if loss_acc).
// `l` is the workspace layout (wide_ws of the largest token count the
// workspace was sized for, >= a.n); tokens are taken in chunks of l.ct.
int wide_grad(const void* K, const void* Vp, const float* theta, const MlpArgs& a, int32_t loss, void* ws,
              const WideWs& l, vggt3::ReduceMode mode, float* dst, float lr, float* loss_out, int loss_acc,
              hipStream_t s) {
  namespace w = vggt3::wide;
  const int64_t nchunks = (a.n + l.ct - 1) / l.ct;
  char* base = static_cast<char*>(ws);
  auto bf = [&](size_t off) { return reinterpret_cast<uint16_t*>(base + off); };
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  const int d = w::kD, m = w::kM;
  const bool dot = loss == VGGT3_LOSS_DOT;
  int rc = check_hip(w::launch_pack(theta, bf(l.wgu), bf(l.wdt), bf(l.wdn), d, m, s), "pack launch");
  if (rc) return rc;
  const float lscale = dot ? -1.0f : 1.0f / d;
  const uint16_t* Kb = static_cast<const uint16_t*>(K);
  const uint16_t* Vb = static_cast<const uint16_t*>(Vp);
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t t0 = c * l.ct, nc = a.n - t0 < l.ct ? a.n - t0 : l.ct;
    const uint16_t* Kc = Kb + t0 * d;
    const uint16_t* Vc = Vb + t0 * d;
    float* lossc = f32(l.loss);
    w::GemmArgs g{};
    // P1: [G | U] = K [W_g | W_u] -> H, A, GP
    g.M = nc; g.N = 2 * m; g.K = d; g.nseg = 1; g.S = 1;
    g.A[0] = Kc; g.lda[0] = d; g.B[0] = bf(l.wgu); g.ldb[0] = d;
    g.out0 = bf(l.h); g.out1 = bf(l.a); g.out2 = bf(l.gp); g.ldo = m;
    rc = check_hip(w::launch_gemm(w::EPI_SWIGLU, g, s), "wide gemm P1");
    if (rc) return rc;
    if (!dot) {
      // P2: Y = H W_d -> -Y, loss partials
      g = w::GemmArgs{};
      g.M = nc; g.N = d; g.K = m; g.nseg = 1; g.S = 1;
      g.A[0] = bf(l.h); g.lda[0] = m; g.B[0] = bf(l.wdt); g.ldb[0] = m;
      g.out0 = bf(l.y); g.ldo = d; g.in0 = Vc; g.ldi = d; g.fout = lossc;
      rc = check_hip(w::launch_gemm(w::EPI_Y_LOSS, g, s), "wide gemm P2");
      if (rc) return rc;
    }
    // P3: D = [-Y | V'] [W_d ; W_d]^T (dot: D = V' W_d^T) -> [dG | dU]
    g = w::GemmArgs{};
    g.M = nc; g.N = m; g.K = d; g.S = 1;
    if (dot) {
      g.nseg = 1; g.A[0] = Vc; g.lda[0] = d; g.B[0] = bf(l.wdn); g.ldb[0] = d;
    } else {
      g.nseg = 2;
      g.A[0] = bf(l.y); g.lda[0] = d; g.A[1] = Vc; g.lda[1] = d;
      g.B[0] = bf(l.wdn); g.ldb[0] = d; g.B[1] = bf(l.wdn); g.ldb[1] = d;
    }
    g.in0 = bf(l.gp); g.in1 = bf(l.a); g.out0 = bf(l.dgu); g.ldo = 2 * m;
    rc = check_hip(w::launch_gemm(w::EPI_DH, g, s), "wide gemm P3");
    if (rc) return rc;
    if (loss_out && !dot) {
      // this chunk's per-workgroup sums of (Y - V')^2 from P2
      const int64_t nt = (nc + w::kTile - 1) / w::kTile * (d / w::kTile);
      rc = check_hip(w::launch_sum(lossc, nt, lscale, c > 0 ? 1 : loss_acc, loss_out, s), "loss sum launch");
      if (rc) return rc;
    }
    // P4: [gW_g | gW_u] += K^T [dG | dU];  gW_d += H^T (-Y) + H^T V' (dot: H^T V')
    g = w::GemmArgs{};
    g.M = d; g.N = 2 * m; g.K = nc; g.nseg = 1; g.S = w::kSplit;
    g.A[0] = Kc; g.lda[0] = d; g.B[0] = bf(l.dgu); g.ldb[0] = 2 * m;
    g.a_rows[0] = nc; g.b_rows[0] = l.ctp;  // [dG | dU] rows nc .. ctp are zeros
    g.fout = f32(l.pgu); g.accumulate = c > 0;
    rc = check_hip(w::launch_gemm(w::EPI_PARTIAL, g, s), "wide gemm P4a");
    if (rc) return rc;
    g = w::GemmArgs{};
    g.M = m; g.N = d; g.K = nc; g.S = w::kSplit;
    // H rows nc .. ctp are zeros
    if (dot) {
      g.nseg = 1; g.A[0] = bf(l.h); g.lda[0] = m; g.B[0] = Vc; g.ldb[0] = d;
      g.a_rows[0] = l.ctp; g.b_rows[0] = nc;
    } else {
      g.nseg = 2;
      g.A[0] = bf(l.h); g.lda[0] = m; g.A[1] = bf(l.h); g.lda[1] = m;
      g.B[0] = bf(l.y); g.ldb[0] = d; g.B[1] = Vc; g.ldb[1] = d;
      g.a_rows[0] = g.a_rows[1] = l.ctp; g.b_rows[0] = g.b_rows[1] = nc;
    }
    g.fout = f32(l.pd); g.accumulate = c > 0;
    rc = check_hip(w::launch_gemm(w::EPI_PARTIAL, g, s), "wide gemm P4b");
    if (rc) return rc;
  }
  const float gscale = dot ? -1.0f : -2.0f / d;
  // dot loss = <W_d, gW_d> (theta read before the update)
  float* wd_dot = (dot && loss_out) ? f32(l.loss) : nullptr;
  rc = check_hip(w::launch_reduce_partials(f32(l.pgu), f32(l.pd), w::kSplit, d, m, gscale, (int)mode, dst, lr,
                                           theta, wd_dot, s),
                 "wide reduce launch");
  if (!rc && wd_dot)
    rc = check_hip(w::launch_sum(wd_dot, w::reduce_blocks(d, m), 1.0f, loss_acc, loss_out, s), "loss sum launch");
  return rc;
}

// Read of the wide MLP: per chunk, H = SwiGLU(Q) then O = H W_d.
int wide_read(const void* Q, const float* theta, void* O, const MlpArgs& a, void* ws, const WideWs& l,
              hipStream_t s) {
  namespace w = vggt3::wide;
  const int64_t nchunks = (a.n + l.ct - 1) / l.ct;
  char* base = static_cast<char*>(ws);
  auto bf = [&](size_t off) { return reinterpret_cast<uint16_t*>(base + off); };
  const int d = w::kD, m = w::kM;
  int rc = check_hip(w::launch_pack(theta, bf(l.wgu), bf(l.wdt), bf(l.wdn), d, m, s), "pack launch");
  if (rc) return rc;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t t0 = c * l.ct, nc = a.n - t0 < l.ct ? a.n - t0 : l.ct;
    w::GemmArgs g{};
    g.M = nc; g.N = 2 * m; g.K = d; g.nseg = 1; g.S = 1;
    g.A[0] = static_cast<const uint16_t*>(Q) + t0 * d; g.lda[0] = d; g.B[0] = bf(l.wgu); g.ldb[0] = d;
    g.out0 = bf(l.h); g.ldo = m;
    rc = check_hip(w::launch_gemm(w::EPI_SWIGLU_H, g, s), "wide gemm R1");
    if (rc) return rc;
    g = w::GemmArgs{};
    g.M = nc; g.N = d; g.K = m; g.nseg = 1; g.S = 1;
    g.A[0] = bf(l.h); g.lda[0] = m; g.B[0] = bf(l.wdt); g.ldb[0] = m;
    g.out0 = static_cast<uint16_t*>(O) + t0 * d; g.ldo = d;
    rc = check_hip(w::launch_gemm(w::EPI_Y_STORE, g, s), "wide gemm R2");
    if (rc) return rc;
  }
  return VGGT3_OK;
}

bool valid_loss(int32_t loss) { return loss == VGGT3_LOSS_MSE || loss == VGGT3_LOSS_DOT; }

// want_loss false: the bf16 kernel skips the loss value (its partials become
// NaN); the fp32 kernel always computes it.
hipError_t launch_partials(const void* K, const void* Vp, const float* theta, const MlpArgs& a, void* ws, int P,
                           int32_t loss, bool want_loss, hipStream_t s) {
  const WsLayout l = ws_layout(a, P);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + l.part);
  float* loss_part = reinterpret_cast<float*>(static_cast<char*>(ws) + l.loss);
  const bool dot = loss == VGGT3_LOSS_DOT;
  if (!f32_kernels(a.dt, a.d, a.m))
    return vggt3::launch_grad_partial_bf16(K, Vp, theta, part, loss_part, a.n, a.H, P, dot, want_loss, s);
  return vggt3::launch_grad_partial_f32(K, Vp, theta, part, loss_part, a.n, a.H, a.d, a.m, P, dot,
                                        a.dt == VGGT3_BF16, s);
}

// Fixed-tree reduce of the workspace's partials in `mode`.
int run_reduce(const MlpArgs& a, void* ws, int P, vggt3::ReduceMode mode, float* dst, float lr, float* loss_out,
               hipStream_t s) {
  const WsLayout l = ws_layout(a, P);
  const float* part = reinterpret_cast<const float*>(static_cast<const char*>(ws) + l.part);
  const float* loss_part = reinterpret_cast<const float*>(static_cast<const char*>(ws) + l.loss);
  return check_hip(vggt3::launch_reduce(part, loss_part, a.H, P, 3 * a.d * a.m, mode, dst, lr, loss_out, s),
                   "reduction kernel launch");
}

// Gradient over all tokens into (part, loss_part) then reduce in `mode`.
int run_grad(const void* K, const void* Vp, const float* theta, const MlpArgs& a, void* ws, int P, int32_t loss,
             vggt3::ReduceMode mode, float* dst, float lr, float* loss_out, hipStream_t s) {
  int rc = check_hip(launch_partials(K, Vp, theta, a, ws, P, loss, loss_out != nullptr, s),
                     "gradient kernel launch");
  if (rc) return rc;
  return run_reduce(a, ws, P, mode, dst, lr, loss_out, s);
}

// Divisor for v_mul_hi division of values below 2^16 (0 stands for 1).
uint32_t div_magic(uint32_t d) { return d == 1 ? 0u : (uint32_t)(((1ull << 32) + d - 1) / d); }

int check_workspace(const MlpArgs& a, const void* ws, size_t ws_bytes, int* P) {
  const size_t need = workspace_bytes(a, P);
  if (need == 0) return VGGT3_OK;
  if (ws == nullptr) return fail(VGGT3_EWORKSPACE, "workspace is NULL, %zu bytes needed", need);
  if (ws_bytes < need) return fail(VGGT3_EWORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(VGGT3_EINVAL, "workspace is not 16-byte aligned");
  return VGGT3_OK;
}

// Events for one streamed call. Destroying an event whose recorded work is
// still pending is allowed: the runtime releases it once that work completes.
struct CallEvents {
  static constexpr int kMax = 8;
  hipEvent_t e[kMax] = {};
  int n = 0;
  hipError_t create(int count) {
    for (; n < count && n < kMax; ++n) {
      const hipError_t r = hipEventCreateWithFlags(&e[n], hipEventDisableTiming);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
  ~CallEvents() {
    for (int i = 0; i < n; ++i) (void)hipEventDestroy(e[i]);
  }
};

// One staging slot holds one chunk of one token tensor.
size_t stage_slot_bytes(int64_t chunk_tokens, int32_t C, int32_t dt) {
  return round256((size_t)chunk_tokens * C * elem_size(dt));
}

// Arguments of a write call other than its workspace (host-side only).
int check_write_args(const MlpArgs& a, const void* K, const void* Vp, const float* theta, float lr, int32_t steps,
                     int32_t loss, int32_t optimizer, int32_t ns_steps, const float* loss_out) {
  int rc = check_mlp(a);
  if (rc) return rc;
  if (!valid_loss(loss)) return fail(VGGT3_EINVAL, "unknown loss %d", loss);
  if (optimizer != VGGT3_OPT_GD && optimizer != VGGT3_OPT_MUON)
    return fail(VGGT3_EINVAL, "unknown optimizer %d", optimizer);
  if (optimizer == VGGT3_OPT_MUON && (ns_steps < 0 || ns_steps > VGGT3_MAX_NS_STEPS))
    return fail(VGGT3_EINVAL, "ns_steps = %d outside [0, %d]", ns_steps, VGGT3_MAX_NS_STEPS);
  if (!std::isfinite(lr)) return fail(VGGT3_EINVAL, "lr is not finite");
  if (steps < 1) return fail(VGGT3_EINVAL, "steps = %d < 1", steps);
  if (theta == nullptr) return fail(VGGT3_EINVAL, "theta is NULL");
  if (!aligned16(theta) || (loss_out && !aligned16(loss_out)))
    return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  if (a.n > 0) {
    if (K == nullptr || Vp == nullptr) return fail(VGGT3_EINVAL, "K or V' is NULL");
    if (!aligned16(K) || !aligned16(Vp)) return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  }
  return VGGT3_OK;
}

// Fixed scratch of vggt3_ttt_write_noalloc: one copy per GPU, in the code
// object's device memory, alive until the process ends. In host code the
// name below is only a stand-in; the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[VGGT3_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on its first use).
int scratch_address(void** out) {
  int dev = 0;
  int rc = check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (rc) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(VGGT3_EUNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    rc = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (rc) return rc;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VGGT3_OK;
}

}  // namespace

extern "C" {

int vggt3_version(void) { return 1 * 10000 + 0 * 100 + 0; }

const char* vggt3_status_str(int status) {
  switch (status) {
    case VGGT3_OK: return "ok";
    case VGGT3_EINVAL: return "invalid argument";
    case VGGT3_EUNSUPPORTED: return "unsupported shape or dtype";
    case VGGT3_EWORKSPACE: return "workspace missing or too small";
    case VGGT3_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* vggt3_last_error(void) { return g_last_error.c_str(); }

int vggt3_shortconv_ex(const void* V, void* Vp, const float* w, int64_t n_views, int32_t grid_h, int32_t grid_w,
                       int32_t n_special, int32_t channels, int32_t ksize, int32_t dtype, void* stream) {
  if (ksize != 3 && ksize != 5) return fail(VGGT3_EUNSUPPORTED, "filter size %d is not 3 or 5", ksize);
  if (!valid_dtype(dtype)) return fail(VGGT3_EINVAL, "dtype %d is not VGGT3_BF16 or VGGT3_F32", dtype);
  if (n_views < 0 || grid_h < 1 || grid_w < 1 || n_special < 0 || channels < 1)
    return fail(VGGT3_EINVAL, "bad layout: n_views %lld, grid %dx%d, n_special %d, channels %d",
                (long long)n_views, grid_h, grid_w, n_special, channels);
  const int vec = dtype == VGGT3_BF16 ? 8 : 4;
  if (channels % vec != 0)
    return fail(VGGT3_EUNSUPPORTED, "channels %d is not a multiple of %d", channels, vec);
  if ((int64_t)grid_h * grid_w > (1 << 24) || n_special > (1 << 20))
    return fail(VGGT3_EUNSUPPORTED, "view too large");
  if (grid_w > vggt3::shortconv_max_grid_w())
    return fail(VGGT3_EUNSUPPORTED, "grid_w %d exceeds %d", grid_w, vggt3::shortconv_max_grid_w());
  if (n_views == 0) return ok();
  if (V == nullptr || Vp == nullptr || w == nullptr) return fail(VGGT3_EINVAL, "NULL pointer");
  if (!aligned16(V) || !aligned16(Vp) || !aligned16(w)) return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  const size_t bytes = (size_t)n_views * ((size_t)n_special + (size_t)grid_h * grid_w) * channels * elem_size(dtype);
  if (overlap(V, bytes, Vp, bytes)) return fail(VGGT3_EINVAL, "V' overlaps V (in-place conv is not supported)");
  if (overlap(w, (size_t)channels * ksize * ksize * sizeof(float), Vp, bytes))
    return fail(VGGT3_EINVAL, "V' overlaps w");
  int rc = check_hip(vggt3::launch_shortconv_k(V, Vp, w, n_views, grid_h, grid_w, n_special, channels, ksize,
                                               dtype == VGGT3_BF16, static_cast<hipStream_t>(stream)),
                     "shortconv launch");
  return rc ? rc : ok();
}

int vggt3_shortconv(const void* V, void* Vp, const float* w, int64_t n_views, int32_t grid_h, int32_t grid_w,
                    int32_t n_special, int32_t channels, int32_t dtype, void* stream) {
  return vggt3_shortconv_ex(V, Vp, w, n_views, grid_h, grid_w, n_special, channels, 3, dtype, stream);
}

size_t vggt3_ttt_workspace_bytes(int64_t n_tokens, int32_t n_heads, int32_t d_head, int32_t d_hidden,
                                 int32_t dtype) {
  const MlpArgs a{n_tokens, n_heads, d_head, d_hidden, dtype};
  if (check_mlp(a) != VGGT3_OK) return 0;
  return workspace_bytes(a, nullptr);
}

int vggt3_ttt_write_ex(const void* K, const void* Vp, float* theta, int64_t n_tokens, int32_t n_heads,
                       int32_t d_head, int32_t d_hidden, float lr, int32_t steps, int32_t loss, int32_t optimizer,
                       int32_t ns_steps, int32_t dtype, void* workspace, size_t workspace_bytes_, float* loss_out,
                       void* stream) {
  const MlpArgs a{n_tokens, n_heads, d_head, d_hidden, dtype};
  int rc = check_write_args(a, K, Vp, theta, lr, steps, loss, optimizer, ns_steps, loss_out);
  if (rc) return rc;
  int P = 1;
  rc = check_workspace(a, workspace, workspace_bytes_, &P);
  if (rc) return rc;
  const size_t tb = theta_bytes(a), xb = token_bytes(a);
  const size_t lb = loss_out ? (size_t)steps * n_heads * sizeof(float) : 0;
  if (overlap(theta, tb, K, xb) || overlap(theta, tb, Vp, xb) || overlap(theta, tb, workspace, workspace_bytes_) ||
      overlap(theta, tb, loss_out, lb))
    return fail(VGGT3_EINVAL, "theta overlaps another argument");
  if (overlap(loss_out, lb, workspace, workspace_bytes_) || overlap(loss_out, lb, K, xb) ||
      overlap(loss_out, lb, Vp, xb))
    return fail(VGGT3_EINVAL, "loss_out overlaps another argument");
  if (overlap(workspace, workspace_bytes_, K, xb) || overlap(workspace, workspace_bytes_, Vp, xb))
    return fail(VGGT3_EINVAL, "workspace overlaps K or V'");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.n == 0) {
    if (loss_out) {
      rc = check_hip(vggt3::launch_fill(loss_out, 0.0f, (int64_t)steps * n_heads, s), "fill launch");
      if (rc) return rc;
    }
    return ok();
  }
  if (is_wide(a.d, a.m)) {
    const WideWs l = wide_ws(a.n);
    char* base = static_cast<char*>(workspace);
    float* gw = reinterpret_cast<float*>(base + l.grad);
    for (int st = 0; st < steps; ++st) {
      float* lrow = loss_out ? loss_out + (size_t)st * n_heads : nullptr;
      if (optimizer == VGGT3_OPT_GD) {
        rc = wide_grad(K, Vp, theta, a, loss, workspace, l, vggt3::kApply, theta, lr, lrow, 0, s);
      } else {
        rc = wide_grad(K, Vp, theta, a, loss, workspace, l, vggt3::kStore, gw, 0.0f, lrow, 0, s);
        if (!rc)
          rc = check_hip(vggt3::wide::launch_muon(theta, gw, lr, a.d, a.m, ns_steps,
                                                  reinterpret_cast<float*>(base + l.ns), s),
                         "wide muon launch");
      }
      if (rc) return rc;
    }
    return ok();
  }
  float* gbuf = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws_layout(a, P).grad);
  for (int st = 0; st < steps; ++st) {
    float* lrow = loss_out ? loss_out + (size_t)st * n_heads : nullptr;
    if (optimizer == VGGT3_OPT_GD) {
      rc = run_grad(K, Vp, theta, a, workspace, P, loss, vggt3::kApply, theta, lr, lrow, s);
    } else {
      rc = run_grad(K, Vp, theta, a, workspace, P, loss, vggt3::kStore, gbuf, 0.0f, lrow, s);
      if (!rc)
        rc = check_hip(vggt3::launch_muon_apply(theta, gbuf, lr, a.H, a.d, a.m, ns_steps, s), "muon launch");
    }
    if (rc) return rc;
  }
  return ok();
}

int vggt3_ttt_write(const void* K, const void* Vp, float* theta, int64_t n_tokens, int32_t n_heads, int32_t d_head,
                    int32_t d_hidden, float lr, int32_t steps, int32_t dtype, void* workspace,
                    size_t workspace_bytes_, float* loss_out, void* stream) {
  return vggt3_ttt_write_ex(K, Vp, theta, n_tokens, n_heads, d_head, d_hidden, lr, steps, VGGT3_LOSS_MSE,
                            VGGT3_OPT_GD, 0, dtype, workspace, workspace_bytes_, loss_out, stream);
}

int vggt3_ttt_write_noalloc(const void* K, const void* Vp, float* theta, int64_t n_tokens, int32_t n_heads,
                            int32_t d_head, int32_t d_hidden, float lr, int32_t steps, int32_t loss,
                            int32_t optimizer, int32_t ns_steps, int32_t dtype, float* loss_out, void* stream) {
  const MlpArgs a{n_tokens, n_heads, d_head, d_hidden, dtype};
  int rc = check_write_args(a, K, Vp, theta, lr, steps, loss, optimizer, ns_steps, loss_out);
  if (rc) return rc;
  if (is_wide(a.d, a.m))
    return fail(VGGT3_EUNSUPPORTED, "the %d -> %d -> %d MLP needs a workspace of GBs; use vggt3_ttt_write_ex",
                a.d, a.m, a.d);
  // Every byte of the workspace this call uses is written by its own kernels
  // before it is read (chunk partials, loss partials, reduced gradient), so
  // the scratch needs no clearing between calls.
  const size_t need = workspace_bytes(a, nullptr);
  if (need > (size_t)VGGT3_NOALLOC_SCRATCH_BYTES)
    return fail(VGGT3_EWORKSPACE, "needs %zu bytes of scratch, more than the fixed %zu (fewer heads fit)", need,
                (size_t)VGGT3_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    rc = scratch_address(&ws);
    if (rc) return rc;
  }
  return vggt3_ttt_write_ex(K, Vp, theta, n_tokens, n_heads, d_head, d_hidden, lr, steps, loss, optimizer,
                            ns_steps, dtype, ws, need, loss_out, stream);
}

int vggt3_ttt_write_conv(const void* K, const void* V, const float* conv_w, int64_t n_views, int32_t grid_h,
                         int32_t grid_w, int32_t n_special, float* theta, int32_t n_heads, int32_t d_head,
                         int32_t d_hidden, float lr, int32_t steps, int32_t loss, int32_t optimizer,
                         int32_t ns_steps, void* Vp_out, void* workspace, size_t workspace_bytes_, float* loss_out,
                         void* stream) {
  if (n_views < 0 || grid_h < 1 || grid_w < 1 || n_special < 0)
    return fail(VGGT3_EINVAL, "bad layout: n_views %lld, grid %dx%d, n_special %d", (long long)n_views, grid_h,
                grid_w, n_special);
  const int64_t tpv = (int64_t)n_special + (int64_t)grid_h * grid_w;
  if (tpv + 31 >= (1 << 16))
    return fail(VGGT3_EUNSUPPORTED, "%lld tokens per view; the fused conv takes at most %d", (long long)tpv,
                (1 << 16) - 32);
  if (grid_w > vggt3::conv_fused_max_grid_w())
    return fail(VGGT3_EUNSUPPORTED, "grid_w %d exceeds the fused conv's %d", grid_w, vggt3::conv_fused_max_grid_w());
  if (n_views > ((int64_t)1 << 40) / tpv) return fail(VGGT3_EUNSUPPORTED, "too many tokens");
  const MlpArgs a{n_views * tpv, n_heads, d_head, d_hidden, VGGT3_BF16};
  int rc = check_write_args(a, K, V, theta, lr, steps, loss, optimizer, ns_steps, loss_out);
  if (rc) return rc;
  if (d_head != 64 || d_hidden != 128)
    return fail(VGGT3_EUNSUPPORTED, "the fused conv write takes (d_head, d_hidden) = (64, 128), not (%d, %d)", d_head,
                d_hidden);
  int P = 1;
  rc = check_workspace(a, workspace, workspace_bytes_, &P);
  if (rc) return rc;
  if (a.n > 0) {
    if (conv_w == nullptr) return fail(VGGT3_EINVAL, "conv_w is NULL");
    if (!aligned16(conv_w) || (Vp_out && !aligned16(Vp_out))) return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  }
  const size_t tb = theta_bytes(a), xb = token_bytes(a), wb = (size_t)a.H * a.d * 9 * sizeof(float);
  const size_t lb = loss_out ? (size_t)steps * n_heads * sizeof(float) : 0;
  const size_t vb = Vp_out ? xb : 0;
  const void* ins[] = {K, V, conv_w};
  const size_t inb[] = {xb, xb, wb};
  for (int i = 0; i < 3; ++i) {
    if (overlap(theta, tb, ins[i], inb[i]) || overlap(loss_out, lb, ins[i], inb[i]) ||
        overlap(workspace, workspace_bytes_, ins[i], inb[i]) || overlap(Vp_out, vb, ins[i], inb[i]))
      return fail(VGGT3_EINVAL, "an output overlaps K, V or conv_w");
  }
  if (overlap(theta, tb, workspace, workspace_bytes_) || overlap(theta, tb, loss_out, lb) ||
      overlap(theta, tb, Vp_out, vb) || overlap(loss_out, lb, workspace, workspace_bytes_) ||
      overlap(loss_out, lb, Vp_out, vb) || overlap(Vp_out, vb, workspace, workspace_bytes_))
    return fail(VGGT3_EINVAL, "theta, loss_out, V' and the workspace must not overlap");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.n == 0) {
    if (loss_out) {
      rc = check_hip(vggt3::launch_fill(loss_out, 0.0f, (int64_t)steps * n_heads, s), "fill launch");
      if (rc) return rc;
    }
    return ok();
  }
  vggt3::ConvGeom geo;
  geo.tpv = (int)tpv;
  geo.n_special = n_special;
  geo.grid_h = grid_h;
  geo.grid_w = grid_w;
  geo.magic_tpv = div_magic((uint32_t)tpv);
  geo.magic_gw = div_magic((uint32_t)grid_w);
  const WsLayout l = ws_layout(a, P);
  char* base = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(base + l.part);
  float* loss_part = reinterpret_cast<float*>(base + l.loss);
  float* gbuf = reinterpret_cast<float*>(base + l.grad);
  const bool dot = loss == VGGT3_LOSS_DOT;
  for (int st = 0; st < steps; ++st) {
    float* lrow = loss_out ? loss_out + (size_t)st * n_heads : nullptr;
    if (st == 0 || Vp_out == nullptr)
      rc = check_hip(vggt3::launch_grad_partial_conv_bf16(K, V, conv_w, st == 0 ? Vp_out : nullptr, geo, theta, part,
                                                          loss_part, a.n, a.H, P, dot, lrow != nullptr, s),
                     "fused conv gradient kernel launch");
    else
      rc = check_hip(vggt3::launch_grad_partial_bf16(K, Vp_out, theta, part, loss_part, a.n, a.H, P, dot,
                                                     lrow != nullptr, s),
                     "gradient kernel launch");
    if (rc) return rc;
    if (optimizer == VGGT3_OPT_GD) {
      rc = run_reduce(a, workspace, P, vggt3::kApply, theta, lr, lrow, s);
    } else {
      rc = run_reduce(a, workspace, P, vggt3::kStore, gbuf, 0.0f, lrow, s);
      if (!rc)
        rc = check_hip(vggt3::launch_muon_apply(theta, gbuf, lr, a.H, a.d, a.m, ns_steps, s), "muon launch");
    }
    if (rc) return rc;
  }
  return ok();
}

int vggt3_ttt_grad_ex(const void* K, const void* Vp, const float* theta, float* grad, int32_t accumulate,
                      int64_t n_tokens, int32_t n_heads, int32_t d_head, int32_t d_hidden, int32_t loss,
                      int32_t dtype, void* workspace, size_t workspace_bytes_, float* loss_out, void* stream) {
  const MlpArgs a{n_tokens, n_heads, d_head, d_hidden, dtype};
  int rc = check_mlp(a);
  if (rc) return rc;
  if (!valid_loss(loss)) return fail(VGGT3_EINVAL, "unknown loss %d", loss);
  if (theta == nullptr || grad == nullptr) return fail(VGGT3_EINVAL, "theta or grad is NULL");
  if (!aligned16(theta) || !aligned16(grad) || (loss_out && !aligned16(loss_out)))
    return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  if (a.n > 0) {
    if (K == nullptr || Vp == nullptr) return fail(VGGT3_EINVAL, "K or V' is NULL");
    if (!aligned16(K) || !aligned16(Vp)) return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  }
  int P = 1;
  rc = check_workspace(a, workspace, workspace_bytes_, &P);
  if (rc) return rc;
  const size_t tb = theta_bytes(a), xb = token_bytes(a);
  const size_t lb = loss_out ? (size_t)n_heads * sizeof(float) : 0;
  if (overlap(grad, tb, theta, tb) || overlap(grad, tb, K, xb) || overlap(grad, tb, Vp, xb) ||
      overlap(grad, tb, workspace, workspace_bytes_) || overlap(grad, tb, loss_out, lb))
    return fail(VGGT3_EINVAL, "grad overlaps another argument");
  if (overlap(loss_out, lb, workspace, workspace_bytes_) || overlap(loss_out, lb, theta, tb))
    return fail(VGGT3_EINVAL, "loss_out overlaps another argument");
  if (overlap(workspace, workspace_bytes_, theta, tb) || overlap(workspace, workspace_bytes_, K, xb) ||
      overlap(workspace, workspace_bytes_, Vp, xb))
    return fail(VGGT3_EINVAL, "workspace overlaps theta, K or V'");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.n == 0) {
    if (!accumulate) {
      rc = check_hip(vggt3::launch_fill(grad, 0.0f, (int64_t)tb / 4, s), "fill launch");
      if (!rc && loss_out) rc = check_hip(vggt3::launch_fill(loss_out, 0.0f, n_heads, s), "fill launch");
      if (rc) return rc;
    }
    return ok();
  }
  if (is_wide(a.d, a.m))
    rc = wide_grad(K, Vp, theta, a, loss, workspace, wide_ws(a.n), accumulate ? vggt3::kAccum : vggt3::kStore, grad,
                   0.0f, loss_out, accumulate ? 1 : 0, s);
  else
    rc = run_grad(K, Vp, theta, a, workspace, P, loss, accumulate ? vggt3::kAccum : vggt3::kStore, grad, 0.0f,
                  loss_out, s);
  return rc ? rc : ok();
}

int vggt3_ttt_grad(const void* K, const void* Vp, const float* theta, float* grad, int32_t accumulate,
                   int64_t n_tokens, int32_t n_heads, int32_t d_head, int32_t d_hidden, int32_t dtype,
                   void* workspace, size_t workspace_bytes_, float* loss_out, void* stream) {
  return vggt3_ttt_grad_ex(K, Vp, theta, grad, accumulate, n_tokens, n_heads, d_head, d_hidden, VGGT3_LOSS_MSE,
                           dtype, workspace, workspace_bytes_, loss_out, stream);
}

int vggt3_ttt_grad_partials_ex(const void* K, const void* Vp, const float* theta, int64_t n_tokens,
                               int32_t n_heads, int32_t d_head, int32_t d_hidden, int32_t loss, int32_t want_loss,
                               int32_t dtype, void* workspace, size_t workspace_bytes_, void* stream) {
  const MlpArgs a{n_tokens, n_heads, d_head, d_hidden, dtype};
  int rc = check_mlp(a);
  if (rc) return rc;
  if (!valid_loss(loss)) return fail(VGGT3_EINVAL, "unknown loss %d", loss);
  if (is_wide(a.d, a.m)) return fail(VGGT3_EUNSUPPORTED, "no per-chunk partials for the %d -> %d MLP", a.d, a.m);
  if (theta == nullptr) return fail(VGGT3_EINVAL, "theta is NULL");
  if (!aligned16(theta)) return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  if (a.n == 0) return ok();
  if (K == nullptr || Vp == nullptr) return fail(VGGT3_EINVAL, "K or V' is NULL");
  if (!aligned16(K) || !aligned16(Vp)) return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  int P = 1;
  rc = check_workspace(a, workspace, workspace_bytes_, &P);
  if (rc) return rc;
  const size_t tb = theta_bytes(a), xb = token_bytes(a);
  if (overlap(workspace, workspace_bytes_, theta, tb) || overlap(workspace, workspace_bytes_, K, xb) ||
      overlap(workspace, workspace_bytes_, Vp, xb))
    return fail(VGGT3_EINVAL, "workspace overlaps another argument");
  rc = check_hip(
      launch_partials(K, Vp, theta, a, workspace, P, loss, want_loss != 0, static_cast<hipStream_t>(stream)),
      "gradient kernel launch");
  return rc ? rc : ok();
}

int vggt3_ttt_grad_partials(const void* K, const void* Vp, const float* theta, int64_t n_tokens, int32_t n_heads,
                            int32_t d_head, int32_t d_hidden, int32_t dtype, void* workspace,
                            size_t workspace_bytes_, void* stream) {
  return vggt3_ttt_grad_partials_ex(K, Vp, theta, n_tokens, n_heads, d_head, d_hidden, VGGT3_LOSS_MSE, 1, dtype,
                                    workspace, workspace_bytes_, stream);
}

int vggt3_ttt_reduce(const void* workspace, size_t workspace_bytes_, int64_t n_tokens, int32_t n_heads,
                     int32_t d_head, int32_t d_hidden, int32_t dtype, int32_t mode, float* dst, float lr,
                     float* loss_out, void* stream) {
  const MlpArgs a{n_tokens, n_heads, d_head, d_hidden, dtype};
  int rc = check_mlp(a);
  if (rc) return rc;
  if (mode != VGGT3_REDUCE_APPLY && mode != VGGT3_REDUCE_STORE && mode != VGGT3_REDUCE_ACCUMULATE)
    return fail(VGGT3_EINVAL, "unknown reduce mode %d", mode);
  if (is_wide(a.d, a.m)) return fail(VGGT3_EUNSUPPORTED, "no per-chunk partials for the %d -> %d MLP", a.d, a.m);
  if (!std::isfinite(lr)) return fail(VGGT3_EINVAL, "lr is not finite");
  if (dst == nullptr) return fail(VGGT3_EINVAL, "dst is NULL");
  if (!aligned16(dst) || (loss_out && !aligned16(loss_out))) return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  const size_t tb = theta_bytes(a);
  const size_t lb = loss_out ? (size_t)n_heads * sizeof(float) : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.n == 0) {
    if (mode == VGGT3_REDUCE_STORE) {
      rc = check_hip(vggt3::launch_fill(dst, 0.0f, (int64_t)tb / 4, s), "fill launch");
      if (!rc && loss_out) rc = check_hip(vggt3::launch_fill(loss_out, 0.0f, n_heads, s), "fill launch");
      if (rc) return rc;
    }
    return ok();
  }
  int P = 1;
  rc = check_workspace(a, workspace, workspace_bytes_, &P);
  if (rc) return rc;
  if (overlap(dst, tb, workspace, workspace_bytes_) || overlap(loss_out, lb, workspace, workspace_bytes_) ||
      overlap(dst, tb, loss_out, lb))
    return fail(VGGT3_EINVAL, "dst or loss_out overlaps another argument");
  const WsLayout l = ws_layout(a, P);
  const float* part = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + l.part);
  const float* loss_part = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + l.loss);
  const vggt3::ReduceMode rm = mode == VGGT3_REDUCE_APPLY   ? vggt3::kApply
                               : mode == VGGT3_REDUCE_STORE ? vggt3::kStore
                                                            : vggt3::kAccum;
  rc = check_hip(vggt3::launch_reduce(part, loss_part, a.H, P, 3 * a.d * a.m, rm, dst, lr, loss_out, s),
                 "reduction kernel launch");
  return rc ? rc : ok();
}

int vggt3_ttt_muon_apply(float* theta, const float* grad, float lr, int32_t n_heads, int32_t d_head,
                         int32_t d_hidden, int32_t ns_steps, void* stream) {
  if (n_heads < 0 || d_head < 1 || d_hidden < 1) return fail(VGGT3_EINVAL, "bad shape");
  if (!((d_head == 64 && d_hidden == 128) || (d_head == 16 && d_hidden == 32)))
    return fail(VGGT3_EUNSUPPORTED, "no Muon kernel for d_head = %d, d_hidden = %d", d_head, d_hidden);
  if (ns_steps < 0 || ns_steps > VGGT3_MAX_NS_STEPS)
    return fail(VGGT3_EINVAL, "ns_steps = %d outside [0, %d]", ns_steps, VGGT3_MAX_NS_STEPS);
  if (!std::isfinite(lr)) return fail(VGGT3_EINVAL, "lr is not finite");
  const int64_t count = (int64_t)n_heads * 3 * d_head * d_hidden;
  if (count == 0) return ok();
  if (theta == nullptr || grad == nullptr) return fail(VGGT3_EINVAL, "theta or grad is NULL");
  if (!aligned16(theta) || !aligned16(grad)) return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  if (overlap(theta, count * 4, grad, count * 4)) return fail(VGGT3_EINVAL, "grad overlaps theta");
  int rc = check_hip(vggt3::launch_muon_apply(theta, grad, lr, n_heads, d_head, d_hidden, ns_steps,
                                              static_cast<hipStream_t>(stream)),
                     "muon launch");
  return rc ? rc : ok();
}

size_t vggt3_ttt_muon_workspace_bytes(int32_t n_heads, int32_t d_head, int32_t d_hidden) {
  if (n_heads != 1 || !is_wide(d_head, d_hidden)) return 0;
  return vggt3::wide::muon_workspace_floats(d_head, d_hidden) * sizeof(float);
}

int vggt3_ttt_muon_apply_ex(float* theta, const float* grad, float lr, int32_t n_heads, int32_t d_head,
                            int32_t d_hidden, int32_t ns_steps, void* workspace, size_t workspace_bytes_,
                            void* stream) {
  if (!is_wide(d_head, d_hidden))
    return vggt3_ttt_muon_apply(theta, grad, lr, n_heads, d_head, d_hidden, ns_steps, stream);
  if (n_heads != 1) return fail(VGGT3_EUNSUPPORTED, "the %d -> %d MLP takes n_heads = 1", d_head, d_hidden);
  if (ns_steps < 0 || ns_steps > VGGT3_MAX_NS_STEPS)
    return fail(VGGT3_EINVAL, "ns_steps = %d outside [0, %d]", ns_steps, VGGT3_MAX_NS_STEPS);
  if (!std::isfinite(lr)) return fail(VGGT3_EINVAL, "lr is not finite");
  if (theta == nullptr || grad == nullptr) return fail(VGGT3_EINVAL, "theta or grad is NULL");
  if (!aligned16(theta) || !aligned16(grad)) return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  const size_t need = vggt3_ttt_muon_workspace_bytes(n_heads, d_head, d_hidden);
  if (workspace == nullptr) return fail(VGGT3_EWORKSPACE, "workspace is NULL, %zu bytes needed", need);
  if (workspace_bytes_ < need) return fail(VGGT3_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes_, need);
  if (!aligned16(workspace)) return fail(VGGT3_EINVAL, "workspace is not 16-byte aligned");
  const size_t tb = (size_t)3 * d_head * d_hidden * sizeof(float);
  if (overlap(theta, tb, grad, tb) || overlap(workspace, workspace_bytes_, theta, tb) ||
      overlap(workspace, workspace_bytes_, grad, tb))
    return fail(VGGT3_EINVAL, "theta, grad and the workspace overlap");
  int rc = check_hip(vggt3::wide::launch_muon(theta, grad, lr, d_head, d_hidden, ns_steps,
                                              static_cast<float*>(workspace), static_cast<hipStream_t>(stream)),
                     "wide muon launch");
  return rc ? rc : ok();
}

int vggt3_ttt_apply(float* theta, const float* grad, float lr, int32_t n_heads, int32_t d_head, int32_t d_hidden,
                    void* stream) {
  if (n_heads < 0 || d_head < 1 || d_hidden < 1) return fail(VGGT3_EINVAL, "bad shape");
  if (!std::isfinite(lr)) return fail(VGGT3_EINVAL, "lr is not finite");
  const int64_t count = (int64_t)n_heads * 3 * d_head * d_hidden;
  if (count == 0) return ok();
  if (theta == nullptr || grad == nullptr) return fail(VGGT3_EINVAL, "theta or grad is NULL");
  if (!aligned16(theta) || !aligned16(grad)) return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  if (overlap(theta, count * 4, grad, count * 4)) return fail(VGGT3_EINVAL, "grad overlaps theta");
  int rc = check_hip(vggt3::launch_apply(theta, grad, lr, count, static_cast<hipStream_t>(stream)), "apply launch");
  return rc ? rc : ok();
}

int vggt3_ttt_read(const void* Q, const float* theta, void* O, int64_t n_tokens, int32_t n_heads, int32_t d_head,
                   int32_t d_hidden, int32_t dtype, void* stream) {
  const MlpArgs a{n_tokens, n_heads, d_head, d_hidden, dtype};
  int rc = check_mlp(a);
  if (rc) return rc;
  if (is_wide(a.d, a.m))
    return fail(VGGT3_EUNSUPPORTED, "the %d -> %d MLP needs a workspace: use vggt3_ttt_read_ex", a.d, a.m);
  if (a.n == 0) return ok();
  if (Q == nullptr || theta == nullptr || O == nullptr) return fail(VGGT3_EINVAL, "NULL pointer");
  if (!aligned16(Q) || !aligned16(theta) || !aligned16(O)) return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  const size_t tb = theta_bytes(a), xb = token_bytes(a);
  if (overlap(O, xb, Q, xb) || overlap(O, xb, theta, tb)) return fail(VGGT3_EINVAL, "O overlaps Q or theta");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_read_any(Q, theta, O, a.n, a.H, a.d, a.m, dtype, s);
  rc = check_hip(e, "read kernel launch");
  return rc ? rc : ok();
}

size_t vggt3_ttt_read_workspace_bytes(int64_t n_tokens, int32_t n_heads, int32_t d_head, int32_t d_hidden,
                                      int32_t dtype) {
  const MlpArgs a{n_tokens, n_heads, d_head, d_hidden, dtype};
  if (check_mlp(a) != VGGT3_OK || a.n == 0 || !is_wide(a.d, a.m)) return 0;
  return wide_ws(a.n).read_total;
}

int vggt3_ttt_read_ex(const void* Q, const float* theta, void* O, int64_t n_tokens, int32_t n_heads, int32_t d_head,
                      int32_t d_hidden, int32_t dtype, void* workspace, size_t workspace_bytes_, void* stream) {
  const MlpArgs a{n_tokens, n_heads, d_head, d_hidden, dtype};
  int rc = check_mlp(a);
  if (rc) return rc;
  if (!is_wide(a.d, a.m))
    return vggt3_ttt_read(Q, theta, O, n_tokens, n_heads, d_head, d_hidden, dtype, stream);
  if (a.n == 0) return ok();
  if (Q == nullptr || theta == nullptr || O == nullptr) return fail(VGGT3_EINVAL, "NULL pointer");
  if (!aligned16(Q) || !aligned16(theta) || !aligned16(O)) return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  const size_t need = wide_ws(a.n).read_total;
  if (workspace == nullptr) return fail(VGGT3_EWORKSPACE, "workspace is NULL, %zu bytes needed", need);
  if (workspace_bytes_ < need) return fail(VGGT3_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes_, need);
  if (!aligned16(workspace)) return fail(VGGT3_EINVAL, "workspace is not 16-byte aligned");
  const size_t tb = theta_bytes(a), xb = token_bytes(a);
  if (overlap(O, xb, Q, xb) || overlap(O, xb, theta, tb) || overlap(O, xb, workspace, workspace_bytes_))
    return fail(VGGT3_EINVAL, "O overlaps Q, theta or the workspace");
  if (overlap(workspace, workspace_bytes_, Q, xb) || overlap(workspace, workspace_bytes_, theta, tb))
    return fail(VGGT3_EINVAL, "workspace overlaps Q or theta");
  rc = wide_read(Q, theta, O, a, workspace, wide_ws(a.n), static_cast<hipStream_t>(stream));
  return rc ? rc : ok();
}

size_t vggt3_ttt_stream_stage_bytes(int64_t chunk_tokens, int32_t n_heads, int32_t d_head, int32_t dtype) {
  if (chunk_tokens < 1 || n_heads < 1 || d_head < 1 || !valid_dtype(dtype)) return 0;
  if ((int64_t)n_heads * d_head > (int64_t)1 << 20) return 0;
  return 4 * stage_slot_bytes(chunk_tokens, n_heads * d_head, dtype);
}

int vggt3_ttt_write_streamed(const void* K_host, const void* Vp_host, float* theta, int64_t n_tokens,
                             int32_t n_heads, int32_t d_head, int32_t d_hidden, float lr, int32_t steps,
                             int32_t loss, int32_t optimizer, int32_t ns_steps, int32_t dtype,
                             int64_t chunk_tokens, void* stage, size_t stage_bytes, void* workspace,
                             size_t workspace_bytes_, float* loss_out, void* stream, void* copy_stream) {
  const MlpArgs a{n_tokens, n_heads, d_head, d_hidden, dtype};
  int rc = check_mlp(a);
  if (rc) return rc;
  if (!valid_loss(loss)) return fail(VGGT3_EINVAL, "unknown loss %d", loss);
  if (optimizer != VGGT3_OPT_GD && optimizer != VGGT3_OPT_MUON)
    return fail(VGGT3_EINVAL, "unknown optimizer %d", optimizer);
  if (optimizer == VGGT3_OPT_MUON && (ns_steps < 0 || ns_steps > VGGT3_MAX_NS_STEPS))
    return fail(VGGT3_EINVAL, "ns_steps = %d outside [0, %d]", ns_steps, VGGT3_MAX_NS_STEPS);
  if (!std::isfinite(lr)) return fail(VGGT3_EINVAL, "lr is not finite");
  if (steps < 1) return fail(VGGT3_EINVAL, "steps = %d < 1", steps);
  if (chunk_tokens < 1) return fail(VGGT3_EINVAL, "chunk_tokens = %lld < 1", (long long)chunk_tokens);
  const bool wide = is_wide(a.d, a.m);
  if (theta == nullptr) return fail(VGGT3_EINVAL, "theta is NULL");
  if (!aligned16(theta) || (loss_out && !aligned16(loss_out)))
    return fail(VGGT3_EINVAL, "pointer not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t lb = loss_out ? (size_t)steps * n_heads * sizeof(float) : 0;
  if (overlap(theta, theta_bytes(a), loss_out, lb)) return fail(VGGT3_EINVAL, "loss_out overlaps theta");
  if (a.n == 0) {
    if (loss_out) {
      rc = check_hip(vggt3::launch_fill(loss_out, 0.0f, (int64_t)steps * n_heads, s), "fill launch");
      if (rc) return rc;
    }
    return ok();
  }
  if (K_host == nullptr || Vp_host == nullptr) return fail(VGGT3_EINVAL, "K or V' is NULL");
  const int64_t ct = chunk_tokens < a.n ? chunk_tokens : a.n;
  const MlpArgs ca{ct, n_heads, d_head, d_hidden, dtype};
  int P = 1;
  rc = check_workspace(ca, workspace, workspace_bytes_, &P);
  if (rc) return rc;
  const int32_t C = n_heads * d_head;
  const size_t slot = stage_slot_bytes(ct, C, dtype), need = 4 * slot;
  if (stage == nullptr) return fail(VGGT3_EINVAL, "stage is NULL");
  if (stage_bytes < need) return fail(VGGT3_EWORKSPACE, "stage has %zu bytes, %zu needed", stage_bytes, need);
  if (!aligned16(stage)) return fail(VGGT3_EINVAL, "stage is not 16-byte aligned");
  const size_t tb = theta_bytes(a);
  if (overlap(theta, tb, stage, stage_bytes) || overlap(theta, tb, workspace, workspace_bytes_))
    return fail(VGGT3_EINVAL, "theta overlaps stage or workspace");
  if (overlap(stage, stage_bytes, workspace, workspace_bytes_) || overlap(loss_out, lb, stage, stage_bytes) ||
      overlap(loss_out, lb, workspace, workspace_bytes_))
    return fail(VGGT3_EINVAL, "stage, workspace and loss_out overlap");

  // The accumulated gradient sits where the workspace layout of a full chunk
  // puts its reduced gradient; a shorter last chunk has no more partials
  // (ttt_num_chunks grows with n), so its partials end before it. The
  // full-width MLP uses its layout for the chunk capacity throughout.
  const WideWs wl = wide_ws(ct);
  float* gacc = reinterpret_cast<float*>(static_cast<char*>(workspace) + (wide ? wl.grad : ws_layout(ca, P).grad));
  const int64_t nc = (a.n + ct - 1) / ct;
  const int64_t tail = a.n - (nc - 1) * ct;
  if (!wide && ws_layout(MlpArgs{tail, n_heads, d_head, d_hidden, dtype},
                         vggt3::ttt_num_chunks(tail, n_heads, tile_tokens(dtype, d_head, d_hidden)))
                       .grad > ws_layout(ca, P).grad)
    return fail(VGGT3_EUNSUPPORTED, "internal: tail chunk layout exceeds the workspace");

  hipStream_t cs = copy_stream ? static_cast<hipStream_t>(copy_stream) : s;
  CallEvents ev;
  rc = check_hip(ev.create(5), "event create");
  if (rc) return rc;
  hipEvent_t entry = ev.e[0], copied[2] = {ev.e[1], ev.e[2]}, freed[2] = {ev.e[3], ev.e[4]};
  // Staging slots may still be read by earlier work on `stream`.
  rc = check_hip(hipEventRecord(entry, s), "event record");
  if (!rc && cs != s) rc = check_hip(hipStreamWaitEvent(cs, entry, 0), "stream wait");
  if (rc) return rc;

  const size_t row = (size_t)C * elem_size(dtype);
  char* st = static_cast<char*>(stage);
  const bool resident = nc <= 2;  // the whole scene fits in the two slots
  int64_t use = 0;
  for (int step = 0; step < steps; ++step) {
    float* lrow = loss_out ? loss_out + (size_t)step * n_heads : nullptr;
    for (int64_t c = 0; c < nc; ++c, ++use) {
      const int sl = resident ? (int)c : (int)(use & 1);
      const int64_t t0 = c * ct, tn = c + 1 < nc ? ct : tail;
      void* Kd = st + (size_t)(2 * sl) * slot;
      void* Vd = st + (size_t)(2 * sl + 1) * slot;
      if (!resident || step == 0) {
        // Refill slot sl once the chunk that last used it has been consumed.
        if (use >= 2) rc = check_hip(hipStreamWaitEvent(cs, freed[sl], 0), "stream wait");
        if (!rc)
          rc = check_hip(hipMemcpyAsync(Kd, static_cast<const char*>(K_host) + (size_t)t0 * row, (size_t)tn * row,
                                        hipMemcpyHostToDevice, cs),
                         "K copy");
        if (!rc)
          rc = check_hip(hipMemcpyAsync(Vd, static_cast<const char*>(Vp_host) + (size_t)t0 * row, (size_t)tn * row,
                                        hipMemcpyHostToDevice, cs),
                         "V' copy");
        if (!rc && cs != s) {
          rc = check_hip(hipEventRecord(copied[sl], cs), "event record");
          if (!rc) rc = check_hip(hipStreamWaitEvent(s, copied[sl], 0), "stream wait");
        }
        if (rc) return rc;
      }
      const MlpArgs ta{tn, n_heads, d_head, d_hidden, dtype};
      if (wide)
        rc = wide_grad(Kd, Vd, theta, ta, loss, workspace, wl, c == 0 ? vggt3::kStore : vggt3::kAccum, gacc, 0.0f,
                       lrow, c > 0 ? 1 : 0, s);
      else
        rc = run_grad(Kd, Vd, theta, ta, workspace,
                      vggt3::ttt_num_chunks(tn, n_heads, tile_tokens(dtype, d_head, d_hidden)), loss,
                      c == 0 ? vggt3::kStore : vggt3::kAccum, gacc, 0.0f, lrow, s);
      if (!rc && cs != s) rc = check_hip(hipEventRecord(freed[sl], s), "event record");
      if (rc) return rc;
    }
    if (optimizer == VGGT3_OPT_GD)
      rc = check_hip(vggt3::launch_apply(theta, gacc, lr, (int64_t)tb / 4, s), "apply launch");
    else if (wide)
      rc = check_hip(vggt3::wide::launch_muon(theta, gacc, lr, d_head, d_hidden, ns_steps,
                                              reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.ns), s),
                     "wide muon launch");
    else
      rc = check_hip(vggt3::launch_muon_apply(theta, gacc, lr, n_heads, d_head, d_hidden, ns_steps, s),
                     "muon launch");
    if (rc) return rc;
  }
  return ok();
}

int vggt3_ttt_read_streamed_ex(const void* Q_host, const float* theta, void* O_host, int64_t n_tokens,
                               int32_t n_heads, int32_t d_head, int32_t d_hidden, int32_t dtype, int64_t chunk_tokens,
                               void* stage, size_t stage_bytes, void* workspace, size_t workspace_bytes_,
                               void* stream, void* h2d_stream, void* d2h_stream) {
  const MlpArgs a{n_tokens, n_heads, d_head, d_hidden, dtype};
  int rc = check_mlp(a);
  if (rc) return rc;
  if (chunk_tokens < 1) return fail(VGGT3_EINVAL, "chunk_tokens = %lld < 1", (long long)chunk_tokens);
  const bool wide = is_wide(a.d, a.m);
  if (a.n == 0) return ok();
  if (Q_host == nullptr || theta == nullptr || O_host == nullptr) return fail(VGGT3_EINVAL, "NULL pointer");
  if (!aligned16(theta)) return fail(VGGT3_EINVAL, "theta is not 16-byte aligned");
  const size_t xb = token_bytes(a);
  if (overlap(Q_host, xb, O_host, xb)) return fail(VGGT3_EINVAL, "O overlaps Q");
  const int64_t ct = chunk_tokens < a.n ? chunk_tokens : a.n;
  const int32_t C = n_heads * d_head;
  const size_t slot = stage_slot_bytes(ct, C, dtype), need = 4 * slot;
  if (stage == nullptr) return fail(VGGT3_EINVAL, "stage is NULL");
  if (stage_bytes < need) return fail(VGGT3_EWORKSPACE, "stage has %zu bytes, %zu needed", stage_bytes, need);
  if (!aligned16(stage)) return fail(VGGT3_EINVAL, "stage is not 16-byte aligned");
  if (overlap(theta, theta_bytes(a), stage, stage_bytes)) return fail(VGGT3_EINVAL, "stage overlaps theta");
  const WideWs wl = wide_ws(ct);
  if (wide) {
    if (workspace == nullptr) return fail(VGGT3_EWORKSPACE, "workspace is NULL, %zu bytes needed", wl.read_total);
    if (workspace_bytes_ < wl.read_total)
      return fail(VGGT3_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes_, wl.read_total);
    if (!aligned16(workspace)) return fail(VGGT3_EINVAL, "workspace is not 16-byte aligned");
    if (overlap(workspace, workspace_bytes_, stage, stage_bytes) ||
        overlap(workspace, workspace_bytes_, theta, theta_bytes(a)))
      return fail(VGGT3_EINVAL, "workspace overlaps stage or theta");
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStream_t hs = h2d_stream ? static_cast<hipStream_t>(h2d_stream) : s;
  hipStream_t ds = d2h_stream ? static_cast<hipStream_t>(d2h_stream) : s;
  CallEvents ev;
  rc = check_hip(ev.create(7), "event create");
  if (rc) return rc;
  hipEvent_t entry = ev.e[0], q_in[2] = {ev.e[1], ev.e[2]}, done[2] = {ev.e[3], ev.e[4]},
             o_out[2] = {ev.e[5], ev.e[6]};
  rc = check_hip(hipEventRecord(entry, s), "event record");
  if (!rc && hs != s) rc = check_hip(hipStreamWaitEvent(hs, entry, 0), "stream wait");
  if (!rc && ds != s && ds != hs) rc = check_hip(hipStreamWaitEvent(ds, entry, 0), "stream wait");
  if (rc) return rc;

  const size_t row = (size_t)C * elem_size(dtype);
  char* st = static_cast<char*>(stage);
  const int64_t nc = (a.n + ct - 1) / ct;
  auto chunk_len = [&](int64_t c) { return c + 1 < nc ? ct : a.n - c * ct; };
  auto q_slot = [&](int64_t c) { return st + (size_t)(2 * (c & 1)) * slot; };
  auto o_slot = [&](int64_t c) { return st + (size_t)(2 * (c & 1) + 1) * slot; };
  // Copy chunk c's queries in once the read of chunk c-2 (same slot) is done.
  auto fetch = [&](int64_t c) -> int {
    int r = VGGT3_OK;
    if (c >= 2 && hs != s) r = check_hip(hipStreamWaitEvent(hs, done[c & 1], 0), "stream wait");
    if (!r)
      r = check_hip(hipMemcpyAsync(q_slot(c), static_cast<const char*>(Q_host) + (size_t)(c * ct) * row,
                                   (size_t)chunk_len(c) * row, hipMemcpyHostToDevice, hs),
                    "Q copy");
    if (!r && hs != s) r = check_hip(hipEventRecord(q_in[c & 1], hs), "event record");
    return r;
  };
  rc = fetch(0);
  if (rc) return rc;
  for (int64_t c = 0; c < nc; ++c) {
    if (c + 1 < nc) {
      rc = fetch(c + 1);
      if (rc) return rc;
    }
    const int sl = (int)(c & 1);
    if (hs != s) rc = check_hip(hipStreamWaitEvent(s, q_in[sl], 0), "stream wait");
    // The O slot is rewritten once chunk c-2's output has left it.
    if (!rc && c >= 2 && ds != s) rc = check_hip(hipStreamWaitEvent(s, o_out[sl], 0), "stream wait");
    if (rc) return rc;
    const int64_t tn = chunk_len(c);
    if (wide) {
      rc = wide_read(q_slot(c), theta, o_slot(c), MlpArgs{tn, n_heads, d_head, d_hidden, dtype}, workspace, wl, s);
    } else {
      hipError_t e = launch_read_any(q_slot(c), theta, o_slot(c), tn, n_heads, d_head, d_hidden, dtype, s);
      rc = check_hip(e, "read kernel launch");
    }
    if (!rc) rc = check_hip(hipEventRecord(done[sl], s), "event record");
    if (!rc && ds != s) rc = check_hip(hipStreamWaitEvent(ds, done[sl], 0), "stream wait");
    if (!rc)
      rc = check_hip(hipMemcpyAsync(static_cast<char*>(O_host) + (size_t)(c * ct) * row, o_slot(c),
                                    (size_t)tn * row, hipMemcpyDeviceToHost, ds),
                     "O copy");
    if (!rc && ds != s) rc = check_hip(hipEventRecord(o_out[sl], ds), "event record");
    if (rc) return rc;
  }
  // Later work on `stream` comes after the last copies out.
  if (ds != s) {
    rc = check_hip(hipStreamWaitEvent(s, o_out[(nc - 1) & 1], 0), "stream wait");
    if (!rc && nc >= 2) rc = check_hip(hipStreamWaitEvent(s, o_out[(nc - 2) & 1], 0), "stream wait");
    if (rc) return rc;
  }
  return ok();
}

int vggt3_ttt_read_streamed(const void* Q_host, const float* theta, void* O_host, int64_t n_tokens,
                            int32_t n_heads, int32_t d_head, int32_t d_hidden, int32_t dtype,
                            int64_t chunk_tokens, void* stage, size_t stage_bytes, void* stream,
                            void* h2d_stream, void* d2h_stream) {
  return vggt3_ttt_read_streamed_ex(Q_host, theta, O_host, n_tokens, n_heads, d_head, d_hidden, dtype, chunk_tokens,
                                    stage, stage_bytes, nullptr, 0, stream, h2d_stream, d2h_stream);
}

}  // extern "C"

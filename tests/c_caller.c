/*
 * A plain C caller of the layer's C ABI (include/vggt3.h), linked against
 * libvggt3.so and the HIP runtime only: no Python, no torch.
 *
 *   c_caller validate        argument checks only (touches no GPU); exit 0 if
 *                            every call returns the documented status
 *   c_caller run OUT.bin     the layer on a small scene on the GPU: ShortConv2D,
 *                            a 2-step write, the read. Writes the inputs and
 *                            the outputs to OUT.bin for a host-side check.
 *
 * OUT.bin layout (little-endian): int32 header
 *   [n_views, grid_h, grid_w, n_special, n_heads, d_head, d_hidden, steps]
 * then float32 lr, then K, V, Q (bf16, [n][C] each), w (f32 [C][3][3]),
 * theta0 (f32 [H][3*d*m]), V' (bf16), theta* (f32), O (bf16), loss (f32 [steps][H]).
 *
 * The inputs come from a small xorshift generator (test data only; the layer
 * draws no random numbers).
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "vggt3.h"

static uint32_t rng_state = 0x9E3779B9u;
static float uniform_pm1(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return (float)((rng_state >> 8) * (1.0 / 16777216.0)) * 2.0f - 1.0f;
}

/* fp32 -> bf16, round to nearest even (finite inputs) */
static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static int expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: status %d (%s), expected %d: %s\n", what, got, vggt3_status_str(got), want,
            vggt3_last_error());
    return 1;
  }
  return 0;
}

static int validate(void) {
  int bad = 0;
  void* fake = (void*)(uintptr_t)0x10000;
  void* fake2 = (void*)(uintptr_t)0x20000000;
  float* ft = (float*)(uintptr_t)0x40000000;
  bad |= vggt3_version() < 10000;
  bad |= expect("conv dtype", vggt3_shortconv(fake, fake2, ft, 2, 37, 37, 5, 1024, 7, NULL), VGGT3_EINVAL);
  bad |= expect("conv in place", vggt3_shortconv(fake, fake, ft, 2, 37, 37, 5, 1024, VGGT3_BF16, NULL),
                VGGT3_EINVAL);
  bad |= expect("conv empty", vggt3_shortconv(fake, fake2, ft, 0, 37, 37, 5, 1024, VGGT3_BF16, NULL), VGGT3_OK);
  size_t ws = vggt3_ttt_workspace_bytes(4096, 16, 64, 128, VGGT3_BF16);
  bad |= ws == 0;
  bad |= expect("write steps 0",
                vggt3_ttt_write(fake, fake2, ft, 4096, 16, 64, 128, 0.1f, 0, VGGT3_BF16, (void*)(uintptr_t)0x60000000,
                                ws, NULL, NULL),
                VGGT3_EINVAL);
  bad |= expect("write workspace", vggt3_ttt_write(fake, fake2, ft, 4096, 16, 64, 128, 0.1f, 1, VGGT3_BF16, NULL, 0,
                                                   NULL, NULL),
                VGGT3_EWORKSPACE);
  bad |= expect("write shape", vggt3_ttt_write(fake, fake2, ft, 4096, 16, 32, 128, 0.1f, 1, VGGT3_BF16, NULL, 0, NULL,
                                               NULL),
                VGGT3_EUNSUPPORTED);
  bad |= expect("read alias", vggt3_ttt_read(fake, ft, fake, 4096, 16, 64, 128, VGGT3_BF16, NULL), VGGT3_EINVAL);
  printf("validate: %s\n", bad ? "FAILED" : "ok");
  return bad;
}

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));          \
      return 2;                                                                   \
    }                                                                             \
  } while (0)

#define VG_OK(call)                                                               \
  do {                                                                            \
    int s_ = (call);                                                              \
    if (s_ != VGGT3_OK) {                                                         \
      fprintf(stderr, "%s: %s: %s\n", #call, vggt3_status_str(s_), vggt3_last_error()); \
      return 3;                                                                   \
    }                                                                             \
  } while (0)

static int run(const char* path) {
  const int32_t n_views = 2, gh = 9, gw = 11, ns = 3, H = 4, d = 64, m = 128, steps = 2;
  const float lr = 0.1f;
  const int32_t C = H * d;
  const int64_t n = (int64_t)n_views * (ns + gh * gw);
  const size_t tok = (size_t)n * C, th_n = (size_t)H * 3 * d * m, w_n = (size_t)C * 9;

  uint16_t* hK = malloc(tok * 2);
  uint16_t* hV = malloc(tok * 2);
  uint16_t* hQ = malloc(tok * 2);
  float* hw = malloc(w_n * 4);
  float* hth = malloc(th_n * 4);
  uint16_t* hVp = malloc(tok * 2);
  uint16_t* hO = malloc(tok * 2);
  float* hth1 = malloc(th_n * 4);
  float hloss[2 * 4];
  if (!hK || !hV || !hQ || !hw || !hth || !hVp || !hO || !hth1) return 4;
  for (size_t i = 0; i < tok; ++i) hK[i] = to_bf16(0.25f * uniform_pm1());
  for (size_t i = 0; i < tok; ++i) hV[i] = to_bf16(0.25f * uniform_pm1());
  for (size_t i = 0; i < tok; ++i) hQ[i] = to_bf16(0.25f * uniform_pm1());
  for (size_t i = 0; i < w_n; ++i) hw[i] = 0.4f * uniform_pm1();
  for (size_t i = 0; i < th_n; ++i) hth[i] = 0.05f * uniform_pm1();

  void *K, *V, *Vp, *Q, *O, *ws, *w, *theta, *loss;
  const size_t wsb = vggt3_ttt_workspace_bytes(n, H, d, m, VGGT3_BF16);
  HIP_OK(hipMalloc(&K, tok * 2));
  HIP_OK(hipMalloc(&V, tok * 2));
  HIP_OK(hipMalloc(&Vp, tok * 2));
  HIP_OK(hipMalloc(&Q, tok * 2));
  HIP_OK(hipMalloc(&O, tok * 2));
  HIP_OK(hipMalloc(&w, w_n * 4));
  HIP_OK(hipMalloc(&theta, th_n * 4));
  HIP_OK(hipMalloc(&loss, sizeof(hloss)));
  HIP_OK(hipMalloc(&ws, wsb));
  HIP_OK(hipMemcpy(K, hK, tok * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(V, hV, tok * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(Q, hQ, tok * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(w, hw, w_n * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(theta, hth, th_n * 4, hipMemcpyHostToDevice));

  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  VG_OK(vggt3_shortconv(V, Vp, (const float*)w, n_views, gh, gw, ns, C, VGGT3_BF16, s));
  VG_OK(vggt3_ttt_write(K, Vp, (float*)theta, n, H, d, m, lr, steps, VGGT3_BF16, ws, wsb, (float*)loss, s));
  VG_OK(vggt3_ttt_read(Q, (const float*)theta, O, n, H, d, m, VGGT3_BF16, s));
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(hVp, Vp, tok * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hO, O, tok * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hth1, theta, th_n * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hloss, loss, sizeof(hloss), hipMemcpyDeviceToHost));

  FILE* f = fopen(path, "wb");
  if (!f) return 5;
  const int32_t hdr[8] = {n_views, gh, gw, ns, H, d, m, steps};
  fwrite(hdr, 4, 8, f);
  fwrite(&lr, 4, 1, f);
  fwrite(hK, 2, tok, f);
  fwrite(hV, 2, tok, f);
  fwrite(hQ, 2, tok, f);
  fwrite(hw, 4, w_n, f);
  fwrite(hth, 4, th_n, f);
  fwrite(hVp, 2, tok, f);
  fwrite(hth1, 4, th_n, f);
  fwrite(hO, 2, tok, f);
  fwrite(hloss, 4, (size_t)steps * H, f);
  fclose(f);
  printf("run: %lld tokens, %d heads, loss[0][0] = %g\n", (long long)n, H, hloss[0]);

  hipStreamDestroy(s);
  hipFree(K);
  hipFree(V);
  hipFree(Vp);
  hipFree(Q);
  hipFree(O);
  hipFree(w);
  hipFree(theta);
  hipFree(loss);
  hipFree(ws);
  free(hK);
  free(hV);
  free(hQ);
  free(hw);
  free(hth);
  free(hVp);
  free(hO);
  free(hth1);
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "validate") == 0) return validate();
  if (argc >= 3 && strcmp(argv[1], "run") == 0) return run(argv[2]);
  fprintf(stderr, "usage: %s validate | run OUT.bin\n", argv[0]);
  return 64;
}

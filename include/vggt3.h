/*
 * vggt3.h — C ABI of the MI355X (gfx950) VGG-T^3 test-time-training layer.
 *
 * The layer replaces a global softmax-attention layer by a fast-weight SwiGLU
 * MLP that is fitted to the scene at inference time and then queried:
 *
 *   1. ShortConv2D  V -> V'   (depthwise 3x3 over each view's patch grid)
 *   2. write        theta* = a few gradient-descent steps on
 *                   sum_i (1/d)||T_theta(k_i) - v'_i||^2          (per head)
 *   3. read         o_i = T_theta*(q_i)
 *
 * with T(x) = (silu(x W_g) * (x W_u)) W_d per head (no biases).
 *
 * Sources, cited by page title and section:
 *   [GRAPH] paper-graph summary "VGG-T3: Offline Feed-Forward 3D Reconstruction
 *           at Scale", section 3.4: "The Test-Time Training (TTT) Framework"
 *           (Eq. 3 optimisation, Eq. 4 query), "Non-Linear Spatial Mixing via
 *           ShortConv2D" (+ Appendix A: special tokens skip the conv), "TTT MLP
 *           Architecture and Inner Optimization" (SwiGLU fast weights),
 *           "Large-Scale Inference Strategies" (Eq. 5 minibatch gradient sum,
 *           query mode).
 *   [BLOG]  neteralex.cn "VGG-T^3 3D reconstruction at scale": the Update-then-
 *           Apply use of the layer, the per-minibatch gradient split, query mode
 *           with frozen weights, and the released interface's default of 1 step.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned (the streamed entry points at the end take HOST token tensors,
 *     as they say). The library allocates no device memory and keeps no state
 *     between calls apart from a per-thread last-error string and the fixed
 *     scratch array of vggt3_ttt_write_noalloc (one per GPU, held until the
 *     process ends).
 *   - Token tensors (K, V, V', Q, O) are row-major [n_tokens][C] with
 *     C = n_heads * d_head; head h owns columns h*d_head .. h*d_head+d_head-1.
 *     Within a scene, tokens are grouped by view, and each view is
 *     [n_special special tokens][grid_h*grid_w patch tokens, row-major].
 *   - dtype VGGT3_BF16: token tensors are bfloat16, MLP contractions run on
 *     bf16 MFMA with fp32 accumulation (at the small (16, 32) head shape the
 *     bf16 inputs are widened exactly and the arithmetic is fp32, with O
 *     rounded to bf16). dtype VGGT3_F32: token tensors are float32 and all
 *     arithmetic is fp32.
 *   - Fast weights theta are float32 [n_heads][3*d_head*d_hidden]; per head the
 *     three row-major blocks W_g [d_head][d_hidden], W_u [d_head][d_hidden],
 *     W_d [d_hidden][d_head].
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is enqueued and a negative vggt3_status is returned. Work
 *     is asynchronous on `stream` (a hipStream_t; NULL = default stream);
 *     device faults surface at the caller's next synchronisation.
 *   - Results are deterministic: identical inputs on the same GPU give
 *     bitwise-identical outputs (no atomics; fixed reduction trees).
 *   - Calls that share a workspace must not run concurrently.
 */
#ifndef VGGT3_H
#define VGGT3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  VGGT3_OK = 0,
  VGGT3_EINVAL = -1,       /* null/misaligned/aliased pointer, negative size, bad lr/steps */
  VGGT3_EUNSUPPORTED = -2, /* shape or dtype the library has no kernel for */
  VGGT3_EWORKSPACE = -3,   /* workspace missing or smaller than vggt3_ttt_workspace_bytes */
  VGGT3_EHIP = -4          /* the HIP runtime refused a launch */
};

enum { VGGT3_BF16 = 0, VGGT3_F32 = 1 };

/* Inner loss of the write:
 *   VGGT3_LOSS_MSE  L_h = sum_i (1/d)||T(k_i) - v'_i||^2   (dL/dY = (2/d)(Y - V'))
 *   VGGT3_LOSS_DOT  L_h = -sum_i T(k_i) . v'_i             (dL/dY = -V')
 * The dot form is the pages' own ([GRAPH] "The dot product loss": the dot
 * product is maximised, here written as a loss to minimise). */
enum { VGGT3_LOSS_MSE = 0, VGGT3_LOSS_DOT = 1 };

/* Update rule of one write step:
 *   VGGT3_OPT_GD    theta <- theta - lr * g
 *   VGGT3_OPT_MUON  theta <- theta - lr * NS(g) per head and weight matrix,
 *                   NS = ns_steps iterations of the quintic Newton-Schulz
 *                   orthogonalisation of the Muon optimiser ([GRAPH] "Muon
 *                   optimizer for inner loop": 5 iterations, lr 0.1; the
 *                   iteration and its coefficients 3.4445, -4.7750, 2.0315 are
 *                   those of the named method, Jordan et al. 2024). No momentum. */
enum { VGGT3_OPT_GD = 0, VGGT3_OPT_MUON = 1 };
#define VGGT3_MAX_NS_STEPS 64

/* Library version (major*10000 + minor*100 + patch). */
int vggt3_version(void);

/* Text for a status code; never NULL. */
const char* vggt3_status_str(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* vggt3_last_error(void);

/*
 * ShortConv2D: V' = depthwise 3x3 convolution of each view's patch grid
 * ([GRAPH] "Non-Linear Spatial Mixing via ShortConv2D": reshape the value
 * tokens to (views, H/p, W/p, C), apply one 3x3 filter per channel, flatten
 * back; Appendix A: camera/register tokens are passed through unchanged).
 *
 *   V        [n_views*(n_special+grid_h*grid_w)][channels], dtype
 *   Vp       same shape and dtype; written. Must not overlap V.
 *   w        float32 [channels][3][3]; w[c][a+1][b+1] multiplies the value at
 *            row offset a, column offset b (cross-correlation), zero padding,
 *            stride 1, no bias; the conv never crosses a view boundary.
 *
 * Each patch output is evaluated in float32 as acc = +0; for a = -1..1 (outer),
 * b = -1..1 (inner): acc = fl(acc + fl(w*v)) — separately rounded, never fused;
 * then rounded to bf16 (ties to even) in bf16 mode. Special tokens are copied
 * bit for bit. channels must be a multiple of 8 (bf16) or 4 (f32), and
 * grid_w at most 4096.
 * n_views == 0 is a no-op.
 */
int vggt3_shortconv(const void* V, void* Vp, const float* w, int64_t n_views, int32_t grid_h,
                    int32_t grid_w, int32_t n_special, int32_t channels, int32_t dtype,
                    void* stream);

/*
 * vggt3_shortconv with a k x k filter, ksize 3 or 5 ([GRAPH] "Non-Linear
 * Spatial Mixing via ShortConv2D", Appendix C Table 9: the "V-5" variant uses
 * 5 x 5). w is float32 [channels][ksize][ksize]; w[c][a+r][b+r] (r = ksize/2)
 * multiplies the value at row offset a, column offset b. The evaluation
 * contract is the same with offsets -r..r (row outer, column inner). Other
 * arguments, errors and limits as in vggt3_shortconv. (Table 9's "KV-3"
 * variant is vggt3_shortconv applied to K as well, with its own filters.)
 */
int vggt3_shortconv_ex(const void* V, void* Vp, const float* w, int64_t n_views, int32_t grid_h,
                       int32_t grid_w, int32_t n_special, int32_t channels, int32_t ksize,
                       int32_t dtype, void* stream);

/*
 * Bytes of device workspace vggt3_ttt_write / vggt3_ttt_grad (and their _ex
 * forms) need for this problem: per-chunk fp32 gradient and loss partials of
 * the Eq. 5 split, plus one reduced gradient for Muon steps. Returns 0 for an
 * unsupported shape.
 */
size_t vggt3_ttt_workspace_bytes(int64_t n_tokens, int32_t n_heads, int32_t d_head,
                                 int32_t d_hidden, int32_t dtype);

/*
 * Write (Update): `steps` full-batch gradient-descent steps of the per-head
 * inner loss L_h = sum_i (1/d)||T(k_i) - v'_i||^2 ([GRAPH] Eq. 3 with a squared
 * error; one step = one pass over all n tokens at the current theta, then
 * theta <- theta - lr * dL/dtheta for all three matrices at once).
 *
 *   K, Vp     [n_tokens][C], dtype; read only.
 *   theta     float32 [n_heads][3*d_head*d_hidden]; read and overwritten with
 *             theta*. Must not overlap any other argument.
 *   lr        finite learning rate; steps >= 1 (the released interface's
 *             default is 1, large scenes use 2).
 *   workspace device buffer of at least vggt3_ttt_workspace_bytes(...) bytes
 *             (may be NULL when that is 0).
 *   loss_out  NULL or float32 [steps][n_heads]: the loss at the theta each
 *             step starts from.
 * Supported (d_head, d_hidden): bf16 (64, 128) and (16, 32); f32 (16, 32) and
 * (64, 128); and bf16 (1024, 4096) with n_heads = 1, the pages' full-width MLP ([GRAPH]
 * "TTT MLP Architecture and Inner Optimization": one 1024 -> 4096 -> 1024
 * SwiGLU), with either loss and either update (vggt3_ttt_write_ex). Its
 * workspace holds the intermediates of one chunk of up to 131,072 tokens
 * (about 5.6 GB), split-K gradient partials and the Newton-Schulz scratch;
 * its read needs vggt3_ttt_read_ex.
 * n_tokens == 0 leaves theta unchanged (losses written as 0).
 */
int vggt3_ttt_write(const void* K, const void* Vp, float* theta, int64_t n_tokens,
                    int32_t n_heads, int32_t d_head, int32_t d_hidden, float lr, int32_t steps,
                    int32_t dtype, void* workspace, size_t workspace_bytes, float* loss_out,
                    void* stream);

/*
 * vggt3_ttt_write with a choice of inner loss (VGGT3_LOSS_*) and update rule
 * (VGGT3_OPT_*); vggt3_ttt_write is the MSE / GD case. ns_steps (0 ..
 * VGGT3_MAX_NS_STEPS) is used only with VGGT3_OPT_MUON; loss_out receives the
 * chosen loss. Muon is supported for (d_head, d_hidden) = (64, 128), (16, 32)
 * and (1024, 4096). Other arguments, errors and n_tokens == 0 as in
 * vggt3_ttt_write.
 */
int vggt3_ttt_write_ex(const void* K, const void* Vp, float* theta, int64_t n_tokens, int32_t n_heads,
                       int32_t d_head, int32_t d_hidden, float lr, int32_t steps, int32_t loss,
                       int32_t optimizer, int32_t ns_steps, int32_t dtype, void* workspace,
                       size_t workspace_bytes, float* loss_out, void* stream);

/*
 * vggt3_ttt_write_ex without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. It calls no allocating routine; its
 * workspace is a fixed array of VGGT3_NOALLOC_SCRATCH_BYTES in the library's
 * device memory, one per GPU (resident from the library's first use on that
 * GPU until the process ends), located once per device.
 *   - Limit: calls whose workspace (vggt3_ttt_workspace_bytes) exceeds
 *     VGGT3_NOALLOC_SCRATCH_BYTES return VGGT3_EWORKSPACE; the 64 MiB hold any
 *     token count at up to 16 heads of the (64, 128) MLP. The full-width
 *     (1024, 4096) MLP returns VGGT3_EUNSUPPORTED.
 *   - All calls on one GPU share that GPU's array: calls that may run at the
 *     same time on one GPU (other host threads, other streams) race and must
 *     be serialised by the caller. Nothing in the array needs clearing: each
 *     call writes every byte it reads.
 * Results are bitwise those of vggt3_ttt_write_ex with its own workspace.
 */
#define VGGT3_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int vggt3_ttt_write_noalloc(const void* K, const void* Vp, float* theta, int64_t n_tokens, int32_t n_heads,
                            int32_t d_head, int32_t d_hidden, float lr, int32_t steps, int32_t loss,
                            int32_t optimizer, int32_t ns_steps, int32_t dtype, float* loss_out,
                            void* stream);

/*
 * Write with the ShortConv2D fused into every gradient pass ([GRAPH] "Non-
 * Linear Spatial Mixing via ShortConv2D" and Appendix A feed the write with
 * V' = conv(V); here V' is formed tile by tile inside the gradient kernel, so
 * it need not exist in device memory).
 *
 *   K, V      [n_views*(n_special+grid_h*grid_w)][C], bf16; read only. V is
 *             the unconvolved value tensor.
 *   conv_w    float32 [C][3][3], as w of vggt3_shortconv.
 *   Vp_out    NULL, or [n_tokens][C] bf16: then the first step also writes
 *             V' there (bitwise the output of vggt3_shortconv) and later steps
 *             read it instead of recomputing it. Must not overlap any other
 *             argument.
 * theta, lr, steps, loss, optimizer, ns_steps, workspace (sized by
 * vggt3_ttt_workspace_bytes(n_tokens, n_heads, 64, 128, VGGT3_BF16)) and
 * loss_out as in vggt3_ttt_write_ex. Results are bitwise those of
 * vggt3_shortconv followed by vggt3_ttt_write_ex.
 * Supported: bf16, (d_head, d_hidden) = (64, 128), grid_w <= 47 (a tile's
 * 3x3 window must fit the kernel's 128-row ring), n_special + grid_h*grid_w
 * <= 65504; other shapes return VGGT3_EUNSUPPORTED. n_views == 0 leaves theta
 * unchanged (losses written as 0).
 * Cost: the conv's vector work adds about as much time to each gradient pass
 * as the separate conv pass takes, so with V' in memory the split path
 * (vggt3_shortconv + vggt3_ttt_write_ex) is as fast or faster; this form
 * saves the n_tokens*C*2 bytes of V'.
 */
int vggt3_ttt_write_conv(const void* K, const void* V, const float* conv_w, int64_t n_views, int32_t grid_h,
                         int32_t grid_w, int32_t n_special, float* theta, int32_t n_heads, int32_t d_head,
                         int32_t d_hidden, float lr, int32_t steps, int32_t loss, int32_t optimizer,
                         int32_t ns_steps, void* Vp_out, void* workspace, size_t workspace_bytes,
                         float* loss_out, void* stream);

/*
 * Gradient of the inner loss at theta over n_tokens tokens ([GRAPH] Eq. 5: the
 * full gradient is the sum of per-minibatch gradients, so chunks of a scene
 * can be fed in any number of calls with accumulate = 1).
 *
 *   grad      float32 [n_heads][3*d_head*d_hidden]; written (accumulate == 0)
 *             or added to (accumulate != 0). Must not overlap theta.
 *   loss_out  NULL or float32 [n_heads], written or added to like grad.
 * Other arguments as in vggt3_ttt_write.
 */
int vggt3_ttt_grad(const void* K, const void* Vp, const float* theta, float* grad,
                   int32_t accumulate, int64_t n_tokens, int32_t n_heads, int32_t d_head,
                   int32_t d_hidden, int32_t dtype, void* workspace, size_t workspace_bytes,
                   float* loss_out, void* stream);

/* vggt3_ttt_grad for either inner loss (VGGT3_LOSS_*). */
int vggt3_ttt_grad_ex(const void* K, const void* Vp, const float* theta, float* grad,
                      int32_t accumulate, int64_t n_tokens, int32_t n_heads, int32_t d_head,
                      int32_t d_hidden, int32_t loss, int32_t dtype, void* workspace,
                      size_t workspace_bytes, float* loss_out, void* stream);

/*
 * The two halves of vggt3_ttt_grad / one step of vggt3_ttt_write, for callers
 * that schedule them themselves (e.g. to exchange per-chunk partials between
 * devices, or to time the gradient pass alone). [GRAPH] Eq. 5 writes the
 * gradient as a sum over minibatches of per-minibatch sums:
 *
 * vggt3_ttt_grad_partials: the per-minibatch sums. Writes one fp32 gradient
 *   partial and one loss partial per (head, token chunk) into `workspace`
 *   (layout private to the library; size from vggt3_ttt_workspace_bytes).
 *   The chunking depends only on (n_tokens, n_heads, dtype).
 *
 * vggt3_ttt_reduce: the sum over minibatches, by a fixed pairwise tree, then
 *   mode VGGT3_REDUCE_APPLY:      dst = theta, theta <- theta - lr * g
 *   mode VGGT3_REDUCE_STORE:      dst = grad,  grad <- g
 *   mode VGGT3_REDUCE_ACCUMULATE: dst = grad,  grad <- grad + g
 *   loss_out (NULL or float32 [n_heads]) receives the loss in the same mode
 *   (APPLY writes it). Arguments (n_tokens, n_heads, d_head, d_hidden, dtype)
 *   must repeat those of the vggt3_ttt_grad_partials call that filled the
 *   workspace. With n_tokens == 0: STORE writes zeros, APPLY and ACCUMULATE
 *   leave dst unchanged.
 */
enum { VGGT3_REDUCE_APPLY = 0, VGGT3_REDUCE_STORE = 1, VGGT3_REDUCE_ACCUMULATE = 2 };

int vggt3_ttt_grad_partials(const void* K, const void* Vp, const float* theta, int64_t n_tokens,
                            int32_t n_heads, int32_t d_head, int32_t d_hidden, int32_t dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/* vggt3_ttt_grad_partials for either inner loss (VGGT3_LOSS_*); the reduce is
 * the same for both. want_loss = 0 skips the loss value: in bf16 the residual
 * is then never formed and the loss partials hold NaN, so a following
 * vggt3_ttt_reduce gives a NaN loss_out (the gradient is unchanged, bit for
 * bit). vggt3_ttt_write and vggt3_ttt_grad do the same when their loss_out is
 * NULL; vggt3_ttt_grad_partials always computes it. */
int vggt3_ttt_grad_partials_ex(const void* K, const void* Vp, const float* theta, int64_t n_tokens,
                               int32_t n_heads, int32_t d_head, int32_t d_hidden, int32_t loss,
                               int32_t want_loss, int32_t dtype, void* workspace, size_t workspace_bytes,
                               void* stream);

int vggt3_ttt_reduce(const void* workspace, size_t workspace_bytes, int64_t n_tokens, int32_t n_heads,
                     int32_t d_head, int32_t d_hidden, int32_t dtype, int32_t mode, float* dst,
                     float lr, float* loss_out, void* stream);

/*
 * Muon update ([GRAPH] "Muon optimizer for inner loop"): for every head and
 * each of its three weight matrices W_g [d][m], W_u [d][m], W_d [m][d]:
 *   theta_W <- theta_W - lr * NS(grad_W),
 * NS(G): X = G / (||G||_F + 1e-7), oriented with rows <= columns (W_d is
 * transposed and back), then ns_steps times A = X X^T, X = a X + (b A + c A A) X
 * with (a, b, c) = (3.4445, -4.7750, 2.0315); all in fp32, deterministic.
 *   theta, grad  float32 [n_heads][3*d_head*d_hidden] (layout of theta); grad
 *                read only and must not overlap theta.
 *   ns_steps     0 .. VGGT3_MAX_NS_STEPS (0 applies the normalised gradient).
 * Supported (d_head, d_hidden): (64, 128) and (16, 32).
 */
int vggt3_ttt_muon_apply(float* theta, const float* grad, float lr, int32_t n_heads, int32_t d_head,
                         int32_t d_hidden, int32_t ns_steps, void* stream);

/*
 * Bytes of device workspace vggt3_ttt_muon_apply_ex needs: 0 for the per-head
 * shapes; for the full-width (1024, 4096) MLP (n_heads = 1) the fp32
 * Newton-Schulz scratch (about 42 MB).
 */
size_t vggt3_ttt_muon_workspace_bytes(int32_t n_heads, int32_t d_head, int32_t d_hidden);

/*
 * vggt3_ttt_muon_apply with a workspace: the only Muon update of the
 * full-width (1024, 4096) MLP (W_g and W_u are 1024 x 4096, W_d 4096 x 1024;
 * the tall W_d is orthogonalised through A = X^T X, X <- a X + X B, the same
 * map on its transpose). The products are fp32 GEMMs. For the per-head shapes
 * the workspace is ignored. theta, grad and the workspace must not overlap.
 */
int vggt3_ttt_muon_apply_ex(float* theta, const float* grad, float lr, int32_t n_heads, int32_t d_head,
                            int32_t d_hidden, int32_t ns_steps, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * One plain gradient-descent update theta <- theta - lr * grad over
 * n_heads*3*d_head*d_hidden float32 values (applies an accumulated gradient,
 * [GRAPH] "Large-Scale Inference Strategies"). grad must not overlap theta.
 */
int vggt3_ttt_apply(float* theta, const float* grad, float lr, int32_t n_heads, int32_t d_head,
                    int32_t d_hidden, void* stream);

/*
 * Read (Apply / query mode): O[i] = T_theta(Q[i]) per head ([GRAPH] Eq. 4;
 * with a frozen theta* this is the query mode for unseen views).
 *
 *   Q         [n_tokens][C], dtype; read only.
 *   theta     float32 [n_heads][3*d_head*d_hidden]; read only.
 *   O         [n_tokens][C], dtype; written. Must not overlap Q or theta.
 * Supported shapes as for vggt3_ttt_write. n_tokens == 0 is a no-op.
 */
int vggt3_ttt_read(const void* Q, const float* theta, void* O, int64_t n_tokens, int32_t n_heads,
                   int32_t d_head, int32_t d_hidden, int32_t dtype, void* stream);

/*
 * Bytes of device workspace vggt3_ttt_read_ex needs: 0 for the per-head
 * shapes; for the full-width (1024, 4096) MLP, bf16 copies of the weights and
 * the hidden activations of one token chunk.
 */
size_t vggt3_ttt_read_workspace_bytes(int64_t n_tokens, int32_t n_heads, int32_t d_head, int32_t d_hidden,
                                      int32_t dtype);

/*
 * vggt3_ttt_read with a workspace (at least vggt3_ttt_read_workspace_bytes);
 * the only read of the full-width (1024, 4096) MLP, which vggt3_ttt_read
 * refuses with VGGT3_EUNSUPPORTED. For the per-head shapes the workspace is
 * ignored. The workspace must not overlap Q, theta or O.
 */
int vggt3_ttt_read_ex(const void* Q, const float* theta, void* O, int64_t n_tokens, int32_t n_heads,
                      int32_t d_head, int32_t d_hidden, int32_t dtype, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Streamed (offloaded) write and read: the scene's token tensors stay in HOST
 * memory and pass through the GPU one chunk of tokens at a time ([GRAPH]
 * "Large-Scale Inference Strategies", single-GPU CPU offloading: load a
 * minibatch to the device, compute its gradient, accumulate, drop it, repeat,
 * then apply the summed update; exact by Eq. 5. Query mode reads a frozen
 * theta* the same way). Host-to-device copies of chunk c+1 run on a copy stream
 * while chunk c is computed on `stream`, through two device staging slots.
 *
 * Host buffers should be pinned (allocated with hipHostMalloc or as pinned
 * tensors) for the copies to run asynchronously; pageable memory gives the
 * same results, with copies that do not overlap the kernels. The caller must
 * not modify or free host inputs, or read host outputs, until `stream` has
 * been synchronised: every copy and kernel of the call is ordered before work
 * enqueued later on `stream`, and after work enqueued earlier on it.
 *
 * Bytes of device staging a streamed call needs for chunks of chunk_tokens
 * tokens: two slots of two token tensors each (K and V' for the write, Q and O
 * for the read). Returns 0 for chunk_tokens < 1 or an invalid shape.
 */
size_t vggt3_ttt_stream_stage_bytes(int64_t chunk_tokens, int32_t n_heads, int32_t d_head, int32_t dtype);

/*
 * vggt3_ttt_write_ex over host-resident K and V'. Each step streams all
 * n_tokens tokens in chunks of chunk_tokens (the last chunk may be shorter):
 * per chunk, the gradient is computed at the step's theta and added into an
 * fp32 accumulator in the workspace; after the last chunk the step's update
 * (VGGT3_OPT_GD or VGGT3_OPT_MUON) is applied. When the whole scene fits in
 * the two staging slots (at most two chunks), it is copied once and reused by
 * every step.
 *
 *   K_host, Vp_host  HOST [n_tokens][C], dtype; read only.
 *   theta            DEVICE float32 [n_heads][3*d_head*d_hidden], updated.
 *   chunk_tokens     >= 1; tokens per device-resident chunk.
 *   stage            DEVICE, at least vggt3_ttt_stream_stage_bytes(
 *                    min(chunk_tokens, n_tokens), ...) bytes.
 *   workspace        DEVICE, at least vggt3_ttt_workspace_bytes(
 *                    min(chunk_tokens, n_tokens), ...) bytes (sized for one
 *                    chunk, not for the scene).
 *   loss_out         NULL or DEVICE float32 [steps][n_heads].
 *   stream           compute stream; copy_stream carries the host-to-device
 *                    copies (NULL or equal to stream serialises them).
 * theta, stage, workspace and loss_out must not overlap. The gradient equals
 * vggt3_ttt_grad called with accumulate on each chunk in turn, bit for bit.
 * The full-width (1, 1024, 4096) MLP is supported too (workspace sized for
 * one chunk the same way; chunks of at most 131,072 tokens keep that workspace
 * at its smallest).
 * Errors as in vggt3_ttt_write_ex; a HIP runtime error part-way through
 * returns VGGT3_EHIP with part of the work enqueued.
 */
int vggt3_ttt_write_streamed(const void* K_host, const void* Vp_host, float* theta, int64_t n_tokens,
                             int32_t n_heads, int32_t d_head, int32_t d_hidden, float lr, int32_t steps,
                             int32_t loss, int32_t optimizer, int32_t ns_steps, int32_t dtype,
                             int64_t chunk_tokens, void* stage, size_t stage_bytes, void* workspace,
                             size_t workspace_bytes, float* loss_out, void* stream, void* copy_stream);

/*
 * vggt3_ttt_read over host-resident Q and O (query mode over a frozen theta*):
 * chunk c+1 is copied in on h2d_stream and chunk c-1 copied out on d2h_stream
 * while chunk c is read on `stream` (the two copy streams may be the same
 * stream; NULL or `stream` serialises the copies with the kernels).
 *
 *   Q_host       HOST [n_tokens][C], dtype; read only.
 *   theta        DEVICE float32 [n_heads][3*d_head*d_hidden]; read only.
 *   O_host       HOST [n_tokens][C], dtype; written. Must not overlap Q_host.
 *   stage        DEVICE, at least vggt3_ttt_stream_stage_bytes(
 *                min(chunk_tokens, n_tokens), ...) bytes; must not overlap
 *                theta.
 * Output equals vggt3_ttt_read's bit for bit. n_tokens == 0 is a no-op.
 */
int vggt3_ttt_read_streamed(const void* Q_host, const float* theta, void* O_host, int64_t n_tokens,
                            int32_t n_heads, int32_t d_head, int32_t d_hidden, int32_t dtype,
                            int64_t chunk_tokens, void* stage, size_t stage_bytes, void* stream,
                            void* h2d_stream, void* d2h_stream);

/*
 * vggt3_ttt_read_streamed with a device workspace of at least
 * vggt3_ttt_read_workspace_bytes(min(chunk_tokens, n_tokens), ...) bytes: the
 * streamed read of the full-width (1024, 4096) MLP. For the per-head shapes
 * the workspace is ignored (and may be NULL). It must not overlap stage or
 * theta.
 */
int vggt3_ttt_read_streamed_ex(const void* Q_host, const float* theta, void* O_host, int64_t n_tokens,
                               int32_t n_heads, int32_t d_head, int32_t d_hidden, int32_t dtype,
                               int64_t chunk_tokens, void* stage, size_t stage_bytes, void* workspace,
                               size_t workspace_bytes, void* stream, void* h2d_stream, void* d2h_stream);

#ifdef __cplusplus
}
#endif

#endif /* VGGT3_H */

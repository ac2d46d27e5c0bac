"""Plain CPU reference of the VGG-T^3 TTT layer (test infrastructure only).

Sources (web pages on VGG-T^3; cited by title and section):
  [BLOG]  neteralex.cn blog post "VGG-T^3 3D reconstruction at scale" — sections on
          writing the scene into an MLP by test-time training (the argmin objective
          and the read o_i = T_theta*(q_i)), on why a plain K->V map is degenerate
          (ShortConv2D on V), and on linear scaling (gradient split over minibatches).
  [GRAPH] paper-graph summary "VGG-T3: Offline Feed-Forward 3D Reconstruction at
          Scale" — section 3.4: "The Test-Time Training (TTT) Framework" (Eq. 3
          optimisation, Eq. 4 query), "Non-Linear Spatial Mixing via ShortConv2D"
          (reshape / 3x3 conv / flatten) with its Appendix A note that camera and
          register tokens skip the conv, "TTT MLP Architecture" (SwiGLU), and
          "Large-Scale Inference Strategies" (Eq. 5 minibatch gradient sum, query mode).

Readings taken where the pages are open (each is listed in the design notes):
  * inner loss: per-token mean squared error over the d outputs, summed over all
    tokens, L_h = sum_i (1/d)||T(k_i) - v'_i||^2, heads independent;
  * optimiser: plain full-batch gradient descent, all three matrices updated
    together from the gradient at the current theta; one step = one full pass;
  * T(x) = (silu(x W_g) * (x W_u)) W_d, no biases, Swish with beta = 1;
  * ShortConv2D: depthwise 3x3 cross-correlation, stride 1, zero padding,
    no bias, one filter per channel, within one view; special tokens copied.

The pages' own inner recipe is also here ([GRAPH] section 3.4, "The dot product
loss" and "Muon optimizer for inner loop"; the Appendix A hyper-parameters):
  * loss="dot": L_h = -sum_i T(k_i) . v'_i (the dot product to be maximised,
    written as a loss to minimise), so dL/dY = -V';
  * opt="muon": each per-head weight-matrix gradient is replaced by its
    Newton-Schulz orthogonalisation (5 iterations of the quintic iteration of
    Jordan et al., 2024, the method the pages name) before theta -= lr * update;
    no momentum and no shape-dependent rescaling (the pages give neither).

Everything here is float64 except ``shortconv``, whose result is defined bit for
bit by a float32 evaluation order (the "conv contract").
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Rounding helpers
# ----------------------------------------------------------------------------


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float32.

    bfloat16 keeps the top 16 bits of an IEEE binary32; rounding adds half an
    ulp of the kept part (0x7FFF plus the kept part's lowest bit, which breaks
    ties towards even) before truncating. NaNs stay NaN.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    out = (r << np.uint64(16)).astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out.reshape(x.shape)


# ----------------------------------------------------------------------------
# ShortConv2D  ([GRAPH] "Non-Linear Spatial Mixing via ShortConv2D"; [BLOG]
# section on the degenerate K->V map)
# ----------------------------------------------------------------------------


def _check_layout(n: int, n_views: int, grid_h: int, grid_w: int, n_special: int) -> int:
    tpv = n_special + grid_h * grid_w
    if n != n_views * tpv:
        raise ValueError(f"{n} tokens do not match {n_views} views x {tpv} tokens")
    return tpv


def shortconv(V, w, n_views: int, grid_h: int, grid_w: int, n_special: int,
              out: str = "bf16") -> np.ndarray:
    """V' = ShortConv2D(V) under the float32 conv contract.

    Each view's patch tokens are reshaped to a (grid_h, grid_w, C) grid, every
    channel c is cross-correlated with its own k x k filter w[c] (k odd: 3 is
    the pages' ShortConv2D, 5 their "V-5" variant of Table 9; zero padding,
    same size) and the grid is flattened back; the view's special tokens are
    copied unchanged.

    Contract (fixes the result bit for bit): per output element the k*k taps
    are visited with the row offset outermost and the column offset innermost,
    both from -k//2 to +k//2; starting from acc = +0.0f, each tap does
    acc = fl32(acc + fl32(w * v)) — a separately rounded float32 product and
    sum, never a fused multiply-add; taps outside the grid see v = 0. With
    ``out="bf16"`` the float32 result is rounded to bfloat16 (ties to even).

    Args: V [n, C] (float32 or exactly-widened bf16 values), w [C, k, k] float32.
    Returns float32 [n, C] (bf16-representable values when out == "bf16").
    """
    V32 = np.asarray(V, dtype=np.float32)
    w32 = np.asarray(w, dtype=np.float32)
    n, C = V32.shape
    k = w32.shape[1]
    if w32.shape != (C, k, k) or k % 2 != 1:
        raise ValueError(f"filters must be [C, k, k] with k odd, got {w32.shape}")
    r = k // 2
    tpv = _check_layout(n, n_views, grid_h, grid_w, n_special)
    res = V32.copy()  # special tokens pass through untouched
    grid = V32.reshape(n_views, tpv, C)[:, n_special:, :].reshape(n_views, grid_h, grid_w, C)
    padded = np.zeros((n_views, grid_h + 2 * r, grid_w + 2 * r, C), dtype=np.float32)
    padded[:, r:r + grid_h, r:r + grid_w, :] = grid
    acc = np.zeros((n_views, grid_h, grid_w, C), dtype=np.float32)
    for dy in range(-r, r + 1):
        for dx in range(-r, r + 1):
            tap = padded[:, r + dy:r + dy + grid_h, r + dx:r + dx + grid_w, :]
            prod = (w32[:, dy + r, dx + r] * tap).astype(np.float32)  # fl32(w * v)
            acc = (acc + prod).astype(np.float32)  # fl32(acc + p)
    if out == "bf16":
        acc = bf16_round(acc)
    elif out != "f32":
        raise ValueError(out)
    res.reshape(n_views, tpv, C)[:, n_special:, :] = acc.reshape(n_views, grid_h * grid_w, C)
    return res


def shortconv_direct(V, w, n_views: int, grid_h: int, grid_w: int, n_special: int) -> np.ndarray:
    """Brute-force depthwise k x k convolution in float64 with explicit loops.

    Written straight from the definition V'[y, x, c] = sum_{a,b in -r..r}
    w[c, a+r, b+r] * V[y+a, x+b, c] (r = k//2) over taps inside the grid. Pure
    Python: tiny inputs only. Used to pin ``shortconv``.
    """
    V64 = np.asarray(V, dtype=np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    n, C = V64.shape
    r = w64.shape[1] // 2
    offs = range(-r, r + 1)
    tpv = _check_layout(n, n_views, grid_h, grid_w, n_special)
    res = V64.copy()
    for v in range(n_views):
        base = v * tpv + n_special
        for y in range(grid_h):
            for x in range(grid_w):
                for c in range(C):
                    s = 0.0
                    for a in offs:
                        for b in offs:
                            yy, xx = y + a, x + b
                            if 0 <= yy < grid_h and 0 <= xx < grid_w:
                                s += w64[c, a + r, b + r] * V64[base + yy * grid_w + xx, c]
                    res[base + y * grid_w + x, c] = s
    return res


# ----------------------------------------------------------------------------
# Fast-weight SwiGLU MLP  ([GRAPH] "TTT MLP Architecture and Inner Optimization")
# ----------------------------------------------------------------------------


def split_theta(theta_h, d: int, m: int):
    """One head's flat parameters -> (W_g [d,m], W_u [d,m], W_d [m,d]), float64."""
    t = np.asarray(theta_h, dtype=np.float64).reshape(-1)
    if t.size != 3 * d * m:
        raise ValueError("theta size")
    return (t[:d * m].reshape(d, m), t[d * m:2 * d * m].reshape(d, m),
            t[2 * d * m:].reshape(m, d))


def join_theta(Wg, Wu, Wd) -> np.ndarray:
    return np.concatenate([np.ravel(Wg), np.ravel(Wu), np.ravel(Wd)])


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def swiglu_forward(X, Wg, Wu, Wd, act: str = "silu") -> dict:
    """T(X) = (act(X W_g) * (X W_u)) W_d with intermediates.

    act = "silu" is the SwiGLU gate silu(g) = g * sigmoid(g). act = "one" makes
    the gate the constant 1 (T(X) = X W_u W_d); it exists only so that tests can
    pin the backward pass against closed forms.
    """
    X = np.asarray(X, dtype=np.float64)
    G = X @ Wg
    U = X @ Wu
    if act == "silu":
        S = _sigmoid(G)
        A = G * S
    elif act == "one":
        S = None
        A = np.ones_like(G)
    else:
        raise ValueError(act)
    H = A * U
    Y = H @ Wd
    return {"G": G, "U": U, "S": S, "A": A, "H": H, "Y": Y}


def head_grad(K, Vp, Wg, Wu, Wd, act: str = "silu", chunk: int = 32768, loss: str = "mse"):
    """Loss and gradient of one head's inner objective at (W_g, W_u, W_d).

    loss="mse": L = sum_i (1/d) ||T(k_i) - v'_i||^2 (Eq. 3 of [GRAPH] with a
    squared-error L_t), dY = (2/d)(Y - V').
    loss="dot": L = -sum_i T(k_i) . v'_i ([GRAPH] "The dot product loss", as a
    quantity to minimise), dY = -V'.
    The gradient is accumulated over fixed token chunks, which Eq. 5 of
    [GRAPH] ("Minibatch gradient decomposition") makes exact. Backward pass by
    the chain rule through T:
        g_Wd = H^T dY, dH = dY W_d^T,
        dU = dH * act(G), dG = dH * U * act'(G), g_Wg = K^T dG, g_Wu = K^T dU,
    with silu'(g) = s (1 + g (1 - s)), s = sigmoid(g).
    Returns (loss, g_Wg, g_Wu, g_Wd), all float64.
    """
    if loss not in ("mse", "dot"):
        raise ValueError(loss)
    K = np.asarray(K)
    Vp = np.asarray(Vp)
    n, d = K.shape
    total = 0.0
    gWg = np.zeros_like(Wg)
    gWu = np.zeros_like(Wu)
    gWd = np.zeros_like(Wd)
    for s in range(0, n, chunk):
        k = np.asarray(K[s:s + chunk], dtype=np.float64)
        v = np.asarray(Vp[s:s + chunk], dtype=np.float64)
        f = swiglu_forward(k, Wg, Wu, Wd, act)
        if loss == "mse":
            R = f["Y"] - v
            total += float(np.sum(R * R)) / d
            dY = (2.0 / d) * R
        else:
            total -= float(np.sum(f["Y"] * v))
            dY = -v
        gWd += f["H"].T @ dY
        dH = dY @ Wd.T
        dU = dH * f["A"]
        if act == "silu":
            S = f["S"]
            dG = dH * f["U"] * (S * (1.0 + f["G"] * (1.0 - S)))
        else:
            dG = np.zeros_like(dH)
        gWg += k.T @ dG
        gWu += k.T @ dU
    return total, gWg, gWu, gWd


def _head_cols(h: int, d: int) -> slice:
    return slice(h * d, (h + 1) * d)


def ttt_grad(K, Vp, theta, n_heads: int, d: int, m: int, act: str = "silu",
             chunk: int = 32768, loss: str = "mse"):
    """Gradient of every head's inner loss at theta: (grad [H, 3dm], loss [H])."""
    theta = np.asarray(theta, dtype=np.float64).reshape(n_heads, 3 * d * m)
    grad = np.zeros_like(theta)
    per_head = np.zeros(n_heads)
    for h in range(n_heads):
        Wg, Wu, Wd = split_theta(theta[h], d, m)
        cols = _head_cols(h, d)
        L, gg, gu, gd = head_grad(K[:, cols], Vp[:, cols], Wg, Wu, Wd, act, chunk, loss)
        grad[h] = join_theta(gg, gu, gd)
        per_head[h] = L
    return grad, per_head


def ttt_loss(K, Vp, theta, n_heads: int, d: int, m: int, act: str = "silu",
             loss: str = "mse") -> np.ndarray:
    """Per-head inner loss at theta (no gradient): sum_i (1/d)||T(k_i) - v'_i||^2
    for loss="mse", -sum_i T(k_i) . v'_i for loss="dot"."""
    theta = np.asarray(theta, dtype=np.float64).reshape(n_heads, 3 * d * m)
    out = np.zeros(n_heads)
    for h in range(n_heads):
        Wg, Wu, Wd = split_theta(theta[h], d, m)
        cols = _head_cols(h, d)
        f = swiglu_forward(np.asarray(K[:, cols], dtype=np.float64), Wg, Wu, Wd, act)
        v = np.asarray(Vp[:, cols], dtype=np.float64)
        if loss == "mse":
            R = f["Y"] - v
            out[h] = float(np.sum(R * R)) / d
        elif loss == "dot":
            out[h] = -float(np.sum(f["Y"] * v))
        else:
            raise ValueError(loss)
    return out


def ttt_apply(theta, grad, lr: float) -> np.ndarray:
    """One plain gradient-descent update theta - lr * grad (all matrices at once)."""
    return np.asarray(theta, dtype=np.float64) - lr * np.asarray(grad, dtype=np.float64)


# Coefficients of the quintic Newton-Schulz iteration of the Muon optimiser
# (Jordan et al., 2024, the method named by [GRAPH] "Muon optimizer for inner
# loop"): X <- a X + (b A + c A^2) X with A = X X^T.
NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_EPS = 1e-7


def newton_schulz(G, steps: int = 5) -> np.ndarray:
    """Approximate orthogonalisation of a matrix by the Muon Newton-Schulz iteration.

    X = G / (||G||_F + eps); a matrix with more rows than columns is handled
    through its transpose (so X X^T is the smaller Gram matrix); then `steps`
    times X <- a X + (b A + c A A) X with A = X X^T. In the singular basis of G
    each step maps every singular value x to p(x) = a x + b x^3 + c x^5.
    """
    a, b, c = NS_COEFFS
    X = np.asarray(G, dtype=np.float64)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = X / (np.linalg.norm(X) + NS_EPS)
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if tall else X


def muon_apply(theta, grad, lr: float, n_heads: int, d: int, m: int, ns_steps: int = 5) -> np.ndarray:
    """theta - lr * NS(g) for each head's W_g, W_u and W_d gradient matrix."""
    theta = np.asarray(theta, dtype=np.float64).reshape(n_heads, 3 * d * m)
    grad = np.asarray(grad, dtype=np.float64).reshape(n_heads, 3 * d * m)
    out = theta.copy()
    for h in range(n_heads):
        gg, gu, gd = split_theta(grad[h], d, m)
        upd = join_theta(newton_schulz(gg, ns_steps), newton_schulz(gu, ns_steps),
                         newton_schulz(gd, ns_steps))
        out[h] = theta[h] - lr * upd
    return out


def ttt_write(K, Vp, theta0, n_heads: int, d: int, m: int, lr: float, steps: int,
              act: str = "silu", reduction: str = "sum", chunk: int = 32768,
              loss: str = "mse", opt: str = "gd", ns_steps: int = 5):
    """Fit the fast weights: `steps` full-batch gradient-descent steps from theta0.

    Eq. 3 of [GRAPH] approximated by a fixed number of plain GD steps; each step
    is one pass over all n tokens at the current theta followed by one update
    with the accumulated gradient ([GRAPH] "Large-Scale Inference Strategies":
    accumulate over minibatches, then apply). ``reduction="mean"`` divides loss
    and gradient by n (an alternative reading kept for tests only). loss="dot"
    and opt="muon" give the pages' own recipe (see the module notes).
    Returns (theta* [H, 3dm], losses [steps, H] at the theta each step starts
    from, grads [steps, H, 3dm]).
    """
    theta = np.asarray(theta0, dtype=np.float64).reshape(n_heads, 3 * d * m).copy()
    n = np.asarray(K).shape[0]
    losses = np.zeros((steps, n_heads))
    grads = np.zeros((steps, n_heads, 3 * d * m))
    for s in range(steps):
        g, L = ttt_grad(K, Vp, theta, n_heads, d, m, act, chunk, loss)
        if reduction == "mean":
            g, L = g / n, L / n
        elif reduction != "sum":
            raise ValueError(reduction)
        losses[s] = L
        grads[s] = g
        if opt == "gd":
            theta = ttt_apply(theta, g, lr)
        elif opt == "muon":
            theta = muon_apply(theta, g, lr, n_heads, d, m, ns_steps)
        else:
            raise ValueError(opt)
    return theta, losses, grads



def ttt_write_offload(K, Vp, theta0, n_heads: int, d: int, m: int, lr: float, steps: int, minibatch: int,
                      act: str = "silu", loss: str = "mse", opt: str = "gd", ns_steps: int = 5):
    """The single-GPU offload schedule of [GRAPH] "Large-Scale Inference
    Strategies": per step, take the tokens one minibatch of `minibatch` tokens
    at a time, compute that minibatch's gradient at the step's theta, add it to
    a running sum, and after the last minibatch apply the summed gradient. By
    Eq. 5 this equals ttt_write up to rounding. Returns (theta* [H, 3dm],
    losses [steps, H]).
    """
    if minibatch < 1:
        raise ValueError("minibatch must be >= 1")
    theta = np.asarray(theta0, dtype=np.float64).reshape(n_heads, 3 * d * m).copy()
    K, Vp = np.asarray(K), np.asarray(Vp)
    n = K.shape[0]
    losses = np.zeros((steps, n_heads))
    for s in range(steps):
        g_sum = np.zeros_like(theta)
        for t0 in range(0, n, minibatch):
            g, L = ttt_grad(K[t0:t0 + minibatch], Vp[t0:t0 + minibatch], theta, n_heads, d, m, act, loss=loss)
            g_sum += g
            losses[s] += L
        if opt == "gd":
            theta = ttt_apply(theta, g_sum, lr)
        elif opt == "muon":
            theta = muon_apply(theta, g_sum, lr, n_heads, d, m, ns_steps)
        else:
            raise ValueError(opt)
    return theta, losses

def ttt_read(Q, theta, n_heads: int, d: int, m: int, act: str = "silu") -> np.ndarray:
    """Read pass o_i = T_theta(q_i) per head (Eq. 4 of [GRAPH]); float64 [n, C]."""
    Q = np.asarray(Q)
    theta = np.asarray(theta, dtype=np.float64).reshape(n_heads, 3 * d * m)
    O = np.zeros((Q.shape[0], n_heads * d))
    for h in range(n_heads):
        Wg, Wu, Wd = split_theta(theta[h], d, m)
        cols = _head_cols(h, d)
        O[:, cols] = swiglu_forward(np.asarray(Q[:, cols], dtype=np.float64), Wg, Wu, Wd, act)["Y"]
    return O

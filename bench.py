"""Benchmark of the VGG-T^3 TTT layer on one MI355X.

One step = one pass of the whole layer over the scene, inputs resident in HBM:
  theta <- theta0; V' = ShortConv2D(V); `steps` x (gradient partials over all
  tokens -> fixed-tree reduce + theta -= lr*g); O = read(Q).
This is exactly the kernel sequence vggt3_ttt_write runs with loss_out = NULL
(the inner-loss value is computed once, untimed, after the timing; --with-loss
times it in every step). The write's two halves are called through the split C
ABI so that the gradient kernel can be bracketed by HIP events on the stream it
runs on.

Prints ONE JSON line (rank 0) with tokens/s over the scene, the roofline of the
dominant kernel (the bf16-MFMA gradient pass), per-phase times, and the CPU
oracle's throughput on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--config views1000]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
SPEC_CLOCK_GHZ = 2.4
PEAK_HBM_GBS = 8000.0
METRIC = "TTT-layer tokens/sec (write+read) at 1000 views; % bf16 MFMA peak"
# The gradient kernel each recipe's timed write steps launch (no loss value).
GRAD_KERNEL = {"mse": "grad_partial_mse_pipe_kernel", "dot": "grad_partial_bf16_kernel<dot>"}
GRAD_SOURCE = os.path.join(ROOT, "test_layer_amd", "csrc", "ttt_write_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grad_partial_bf16_views1000_traffic.json")


RECIPES = {
    # name: (loss, optimizer, description)
    "mse_gd": ("mse", "gd", "mean-squared inner loss, plain gradient descent"),
    "dot_muon": ("dot", "muon", "the pages' recipe: dot-product inner loss, Muon update (5 Newton-Schulz steps)"),
    "dot_gd": ("dot", "gd", "dot-product inner loss, plain gradient descent"),
}


def flops_per_token(cfg, loss="mse"):
    """Algorithmic flops per token: a write step with the squared-error loss is
    7 GEMM passes of 2*d*m per head (G, U, Y forward; dH backward; three weight
    gradients); the dot-product loss needs no Y (dL/dY = -V'), so 6; read = 3."""
    per_gemm = 2 * cfg.d_head * cfg.d_hidden * cfg.n_heads
    return (7 if loss == "mse" else 6) * per_gemm, 3 * per_gemm


def source_sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_counter_record(recipe, config, kernel):
    """The committed rocprofv3 counter record of the gradient kernel for this
    recipe and workload (HBM bytes per launch, and the shader clock the kernel
    ran at: its GPU-active cycles over its event-timed launch on the profiled
    box), or None if there is none, it covers another kernel, or it was taken
    on different kernel source."""
    tag = config if recipe == "mse_gd" else f"{recipe}_{config}"
    path = TRAFFIC_FILE.replace("_views1000", f"_{tag}")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel or rec.get("source_sha256") != source_sha256(GRAD_SOURCE):
        return None
    return rec


def cpu_baseline(inp, cfg, target_s=15.0, max_views=256, loss="mse", opt="gd", views_fixed=0):
    """The fp64 CPU oracle, as it stands, on the first s views of the same
    scene (conv, `steps` write steps over those tokens, read). s doubles from
    2 views until one run takes >= target_s / 2 (or max_views); with
    views_fixed, s is that many views (all of them for the whole scene), run
    once."""
    import numpy as np
    import torch

    import oracle

    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 0) for i in info if i.get("user_api") == "blas"] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    tpv = cfg.tokens_per_view
    w = inp.conv_w.cpu().numpy()
    th0 = inp.theta0.cpu().numpy()
    views = min(views_fixed, cfg.n_views) if views_fixed > 0 else 2
    while True:
        n = views * tpv
        if views_fixed > 0:
            print(f"[cpu baseline] oracle on the first {views} views ({n} tokens)", file=sys.stderr, flush=True)
        K = inp.K[:n].to(torch.float32).cpu().numpy().astype(np.float64)
        V = inp.V[:n].to(torch.float32).cpu().numpy()
        Q = inp.Q[:n].to(torch.float32).cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        Vp = oracle.shortconv(V, w, views, cfg.grid_h, cfg.grid_w, cfg.n_special, out="bf16")
        th, _, _ = oracle.ttt_write(K, Vp.astype(np.float64), th0, cfg.n_heads, cfg.d_head, cfg.d_hidden,
                                    cfg.lr, cfg.steps, loss=loss, opt=opt)
        oracle.ttt_read(Q, th, cfg.n_heads, cfg.d_head, cfg.d_hidden)
        dt = time.perf_counter() - t0
        if views_fixed > 0 or dt >= target_s / 2 or views >= max_views or views * 2 > cfg.n_views:
            break
        views *= 2
    return {
        "value": n / dt,
        "unit": "tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"first {views} views ({n} tokens) of the same scene: fp64 numpy oracle conv + "
                   f"{cfg.steps} write steps + read over those tokens, all {cfg.n_heads} heads; {dt:.2f} s; "
                   f"host {platform.processor() or platform.machine()}, {os.cpu_count()} logical CPUs"),
    }


def offload_bench(tla, inp, Vp, cfg, args, loss_kind, opt_kind):
    """Time the layer with its token tensors in host memory: per step the
    streamed write (every write step re-streams K and V') and the streamed
    read of Q into a host O. V' is precomputed (the conv is not streamed)."""
    import torch

    chunk = args.offload
    n, H = cfg.n_tokens, cfg.n_heads

    def pinned(t):
        h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
        h.copy_(t)
        return h

    Kh, Vh, Qh = pinned(inp.K), pinned(Vp), pinned(inp.Q)
    Oh = torch.empty(Qh.shape, dtype=Qh.dtype, pin_memory=True)
    theta = inp.theta0.clone()
    d, m = cfg.d_head, cfg.d_hidden
    dt_code = tla.BF16 if cfg.dtype == "bf16" else tla.F32
    ct = min(chunk, n)
    stage = torch.empty(tla.stage_bytes(ct, H, d, dt_code), dtype=torch.uint8, device=theta.device)
    ws = tla.make_workspace(ct, H, d, m, dt_code, theta.device)

    def step():
        theta.copy_(inp.theta0)
        tla.ttt_write_streamed(Kh, Vh, theta, cfg.lr, cfg.steps, H, chunk, stage=stage, workspace=ws,
                               loss=loss_kind, optimizer=opt_kind)
        tla.ttt_read_streamed(Qh, theta, H, chunk, out=Oh, stage=stage)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k = max(1, min(args.steps, 3))
    a.record()
    for _ in range(k):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / k

    # the link's own rate: one plain pinned host-to-device and device-to-host copy of 1 GiB
    src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=theta.device)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    a.record()
    dst.copy_(src, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    h2d_gbps = (1 << 30) / (a.elapsed_time(b) * 1e-3) / 1e9
    a.record()
    src.copy_(dst, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    d2h_gbps = (1 << 30) / (a.elapsed_time(b) * 1e-3) / 1e9

    xb = Kh.numel() * Kh.element_size()
    qb = Qh.numel() * Qh.element_size()
    h2d = cfg.steps * 2 * xb + qb if -(-n // ct) > 2 else 2 * xb + qb
    d2h = qb
    return {
        "chunk_tokens": chunk, "ms_per_step": ms, "tokens_per_s": n / (ms * 1e-3), "steps_timed": k,
        "h2d_bytes_per_step": h2d, "d2h_bytes_per_step": d2h,
        "pcie_GBps": (h2d + d2h) / (ms * 1e-3) / 1e9,
        "copy_GBps": {"h2d": h2d_gbps, "d2h": d2h_gbps},
        "note": "K, V' and Q in pinned host memory, O written to pinned host memory; V' precomputed",
    }


def conv_fused_bench(tla, inp, cfg, args, loss_kind, opt_kind, ws, O):
    """Time the layer step with the ShortConv2D fused into the write
    (vggt3_ttt_write_conv) in its two forms, beside the split step:
    "all": every gradient pass forms V' itself (V' never in memory);
    "first": the first pass forms V' and writes it, the second reads it."""
    import torch
    n, H = cfg.n_tokens, cfg.n_heads
    out = {}
    for mode in ("all", "first"):
        theta = inp.theta0.clone()
        Vo = torch.empty_like(inp.V) if mode == "first" else None

        def write():
            theta.copy_(inp.theta0)
            tla.ttt_write_conv(inp.K, inp.V, inp.conv_w, cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special, theta,
                               cfg.lr, cfg.steps, H, Vp_out=Vo, workspace=ws, loss=loss_kind, optimizer=opt_kind)

        for _ in range(args.warmup):
            write()
            tla.ttt_read(inp.Q, theta, H, out=O)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev[3 * i].record()
            write()
            ev[3 * i + 1].record()
            tla.ttt_read(inp.Q, theta, H, out=O)
            ev[3 * i + 2].record()
        torch.cuda.synchronize()
        step_ms = sum(ev[3 * i].elapsed_time(ev[3 * i + 2]) for i in range(args.steps)) / args.steps
        write_ms = sum(ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(args.steps)) / args.steps
        out[mode] = {"ms_per_step": step_ms, "tokens_per_s": n / (step_ms * 1e-3), "conv_and_write_ms": write_ms}
        del Vo
    return out


def wide_bench(args, loss_kind, opt_kind, recipe_desc):
    """The pages' full-width fast-weight MLP (one 1024 -> 4096 -> 1024 SwiGLU
    over the whole token) on the same scene: conv, `steps` write steps through
    vggt3_ttt_write_ex (a chunked sequence of bf16 MFMA GEMMs with fused
    epilogues, then the GD or Muon update), read through vggt3_ttt_read_ex.
    The roofline is that of the write's GEMM sequence as a whole: algorithmic
    gradient flops over the write's event time (the Muon update included)."""
    import dataclasses

    import torch

    import test_layer_amd as tla
    from synth import CONFIGS, make_inputs

    base = CONFIGS[args.config]
    cfg = dataclasses.replace(
        base, name=f"{base.name}_wide", n_heads=1, d_head=1024, d_hidden=4096,
        description=(f"{base.n_views} views = {base.n_tokens:,} tokens, one 1024 -> 4096 -> 1024 SwiGLU fast-weight "
                     f"MLP, {base.steps} steps + full read"))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(cfg, dev)
    n, d, m = cfg.n_tokens, cfg.d_head, cfg.d_hidden
    Vp = torch.empty_like(inp.V)
    O = torch.empty_like(inp.Q)
    theta = inp.theta0.clone()
    ws = tla.make_workspace(n, 1, d, m, tla.BF16, dev)
    rws = torch.empty(tla.read_workspace_bytes(n, 1, d, m, tla.BF16), dtype=torch.uint8, device=dev)
    loss = torch.zeros((cfg.steps, 1), device=dev)

    def step(ev=None):
        theta.copy_(inp.theta0)
        if ev:
            ev[0].record()
        tla.shortconv(inp.V, inp.conv_w, cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special, out=Vp)
        if ev:
            ev[1].record()
        tla.ttt_write(inp.K, Vp, theta, cfg.lr, cfg.steps, 1, workspace=ws, loss_out=loss, loss=loss_kind,
                      optimizer=opt_kind)
        if ev:
            ev[2].record()
        tla.ttt_read(inp.Q, theta, 1, out=O, workspace=rws)
        if ev:
            ev[3].record()

    def mk():
        return torch.cuda.Event(enable_timing=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[mk() for _ in range(4)] for _ in range(args.steps)]
    start, end = mk(), mk()
    start.record()
    for i in range(args.steps):
        step(events[i])
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    conv_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    write_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    read_ms = sum(e[2].elapsed_time(e[3]) for e in events) / args.steps
    fw, fr = flops_per_token(cfg, loss_kind)
    achieved = fw * n * cfg.steps / (write_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": n / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "n_views": cfg.n_views, "tokens_per_view": cfg.tokens_per_view, "n_tokens": n,
            "n_heads": 1, "d_head": d, "d_hidden": m, "write_steps": cfg.steps, "lr": cfg.lr,
            "read_tokens": inp.Q.shape[0], "parallelism": "single GPU", "recipe": f"{args.recipe}: {recipe_desc}",
            "conv_variant": "3x3 on V",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "wide write: per token chunk P1-P4 bf16 GEMMs (gemm_kernel<...>) + reduce",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "clock_GHz_from_counters": None,
            "frac_at_counter_clock": None,
            "traffic": None,
            "avg_launch_ms": write_ms / cfg.steps,
            "flops_per_launch": fw * n,
        },
        "phases_ms": {"conv": conv_ms, "write": write_ms, "read": read_ms},
        "mfma_frac_mlp_contractions": (fw * n * cfg.steps + fr * inp.Q.shape[0]) / ((write_ms + read_ms) * 1e-3)
                                      / 1e12 / PEAK_BF16_TFLOPS,
        "read_TFLOPs": fr * inp.Q.shape[0] / (read_ms * 1e-3) / 1e12,
        "final_loss": float(loss[-1, 0].item()),
    }
    if args.offload > 0:
        res["offload"] = offload_bench(tla, inp, Vp, cfg, args, loss_kind, opt_kind)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, cfg, loss=loss_kind, opt=opt_kind,
                                           views_fixed=args.cpu_baseline_views)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="views1000")
    ap.add_argument("--recipe", default="mse_gd", choices=sorted(RECIPES),
                    help="inner loss and update rule (default: squared error + gradient descent)")
    ap.add_argument("--conv-variant", default="v3", choices=["v3", "v5", "kv3"],
                    help="ShortConv2D variant of the pages' Table 9: 3x3 on V (default), 5x5 on V, 3x3 on K and V")
    ap.add_argument("--mlp", default="per-head", choices=["per-head", "wide"],
                    help="fast-weight MLP: 16 per-head SwiGLUs 64 -> 128 -> 64 (default) or the pages' full-width "
                         "1024 -> 4096 -> 1024 SwiGLU")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-views", type=int, default=0, metavar="S",
                    help="run the CPU oracle baseline once on the first S views (the whole scene if S >= its "
                         "views) instead of the bounded sample of 10-30 s; 1000 views take about 100 s and "
                         "about 60 GB of host memory")
    ap.add_argument("--with-loss", action="store_true",
                    help="compute the inner-loss value in every timed write step (as vggt3_ttt_write with a "
                         "loss_out does); by default it is computed once, after timing")
    ap.add_argument("--offload", type=int, default=0, metavar="CHUNK",
                    help="also time the offloaded step (K, V', Q in pinned host memory, streamed through the GPU in "
                         "CHUNK-token chunks; O streamed back) and report it under 'offload' (never as value)")
    ap.add_argument("--conv-fused", action="store_true",
                    help="also time the step with the ShortConv2D fused into the write (vggt3_ttt_write_conv), "
                         "V' formed in every pass or only in the first, and report it under 'conv_fused'")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on exactly one GPU; multi-GPU runs (--gpus > 1) are not supported "
              "(the layer's data-parallel sharding is a design only, with no multi-GPU code).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import test_layer_amd as tla
    from synth import CONFIGS, make_inputs

    cfg = CONFIGS[args.config]
    loss_kind, opt_kind, recipe_desc = RECIPES[args.recipe]
    if args.mlp == "wide":
        wide_bench(args, loss_kind, opt_kind, recipe_desc)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(cfg, dev)
    n, H, d, m = cfg.n_tokens, cfg.n_heads, cfg.d_head, cfg.d_hidden
    dt_code = tla.BF16 if cfg.dtype == "bf16" else tla.F32
    Vp = torch.empty_like(inp.V)
    conv_w = inp.conv_w
    conv_k = None
    Kp = inp.K
    if args.conv_variant != "v3":
        gen = torch.Generator(device="cpu").manual_seed(cfg.seed * 1_000_003 + 17)
        if args.conv_variant == "v5":
            conv_w = (torch.randn((cfg.channels, 5, 5), generator=gen) / 5).to(dev)
        else:
            conv_k = (torch.randn((cfg.channels, 3, 3), generator=gen) / 3).to(dev)
            Kp = torch.empty_like(inp.K)
    O = torch.empty_like(inp.Q)
    theta = inp.theta0.clone()
    ws = tla.make_workspace(n, H, d, m, dt_code, dev)
    loss = torch.zeros((cfg.steps, H), device=dev)
    gbuf = torch.empty_like(theta)
    nq = inp.Q.shape[0]

    # The timed step computes what vggt3_ttt_write(loss_out = NULL) computes: the
    # inner-loss value is a diagnostic the layer does not need (--with-loss
    # times it too). One untimed step with the loss follows the timing.
    with_loss = args.with_loss

    def step(ev=None):
        theta.copy_(inp.theta0)
        if ev:
            ev["c0"].record()
        tla.shortconv(inp.V, conv_w, cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special, out=Vp)
        if conv_k is not None:
            tla.shortconv(inp.K, conv_k, cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special, out=Kp)
        if ev:
            ev["c1"].record()
        for s in range(cfg.steps):
            if ev:
                ev["g"][s][0].record()
            tla.ttt_grad_partials(Kp, Vp, theta, H, ws, loss=loss_kind, want_loss=with_loss)
            if ev:
                ev["g"][s][1].record()
            lrow = loss[s] if with_loss else None
            if opt_kind == "gd":
                tla.ttt_reduce(ws, n, H, d, m, dt_code, tla.REDUCE_APPLY, theta, cfg.lr, lrow)
            else:
                tla.ttt_reduce(ws, n, H, d, m, dt_code, tla.REDUCE_STORE, gbuf, 0.0, lrow)
                tla.ttt_muon_apply(theta, gbuf, cfg.lr, H, d, m, 5)
            if ev:
                ev["u"][s].record()
        if ev:
            ev["w1"].record()
        tla.ttt_read(inp.Q, theta, H, out=O)
        if ev:
            ev["r1"].record()

    def mk():
        return torch.cuda.Event(enable_timing=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [{"c0": mk(), "c1": mk(), "w1": mk(), "r1": mk(),
               "g": [(mk(), mk()) for _ in range(cfg.steps)], "u": [mk() for _ in range(cfg.steps)]}
              for _ in range(args.steps)]
    start, end = mk(), mk()
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(events[i])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    if not with_loss:
        with_loss = True
        step()
        torch.cuda.synchronize()

    conv_ms = sum(e["c0"].elapsed_time(e["c1"]) for e in events) / args.steps
    write_ms = sum(e["c1"].elapsed_time(e["w1"]) for e in events) / args.steps
    read_ms = sum(e["w1"].elapsed_time(e["r1"]) for e in events) / args.steps
    grad_ms = [a.elapsed_time(b) for e in events for (a, b) in e["g"]]
    grad_avg_ms = sum(grad_ms) / len(grad_ms)
    # The update after each gradient pass: the fixed-tree reduce of the chunk
    # partials plus theta -= lr g (and, for Muon, the Newton-Schulz update).
    upd_ms = [e["g"][s][1].elapsed_time(e["u"][s]) for e in events for s in range(cfg.steps)]
    update_avg_ms = sum(upd_ms) / len(upd_ms)

    fw, fr = flops_per_token(cfg, loss_kind)
    grad_flops = fw * n  # per launch of the gradient kernel
    achieved = grad_flops / (grad_avg_ms * 1e-3) / 1e12
    grad_kernel = (("grad_partial_bf16_kernel" + ("<dot>" if loss_kind == "dot" else "") + " (with loss value)")
                   if args.with_loss else GRAD_KERNEL[loss_kind])
    counter_rec = load_counter_record(args.recipe, cfg.name, grad_kernel)
    clock = counter_rec.get("clock_GHz") if counter_rec else None
    mlp_frac = (fw * n * cfg.steps + fr * nq) / ((write_ms + read_ms) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    esz = 2 if cfg.dtype == "bf16" else 4
    conv_bytes = 2 * n * H * d * esz * (2 if args.conv_variant == "kv3" else 1)
    read_bytes = 2 * nq * H * d * esz
    # Gradient-descent update: the partials (the workspace less its theta-sized
    # gradient buffer and at most 4 KB of loss partials) read once, theta read
    # and written.
    theta_bytes = theta.numel() * theta.element_size()
    update_bytes = (ws.numel() * ws.element_size() - theta_bytes) + 2 * theta_bytes

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    res = {
        "metric": METRIC,
        "value": n / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "n_views": cfg.n_views, "tokens_per_view": cfg.tokens_per_view, "n_tokens": n,
            "n_heads": H, "d_head": d, "d_hidden": m, "write_steps": cfg.steps, "lr": cfg.lr,
            "read_tokens": nq, "parallelism": "single GPU", "recipe": f"{args.recipe}: {recipe_desc}",
            "conv_variant": {"v3": "3x3 on V", "v5": "5x5 on V", "kv3": "3x3 on K and on V"}[args.conv_variant],
        },
        "roofline": {
            "bound": "mfma",
            "kernel": grad_kernel,
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "clock_GHz_from_counters": clock,
            "frac_at_counter_clock": achieved / (PEAK_BF16_TFLOPS * clock / SPEC_CLOCK_GHZ) if clock else None,
            "traffic": counter_rec["traffic_bytes_per_launch"] if counter_rec else None,
            "avg_launch_ms": grad_avg_ms,
            "flops_per_launch": grad_flops,
        },
        "phases_ms": {"conv": conv_ms, "write": write_ms, "read": read_ms, "update_each": update_avg_ms},
        "mfma_frac_mlp_contractions": mlp_frac,
        # Scene tokens through conv + write alone, and the read's own query rate
        # (the query-mode read of unseen views reads fewer tokens than the scene).
        "scene_tokens_per_s_without_read": n / ((conv_ms + write_ms) * 1e-3),
        "read_tokens_per_s": nq / (read_ms * 1e-3),
        "hbm_GBps": {"conv": conv_bytes / (conv_ms * 1e-3) / 1e9, "read": read_bytes / (read_ms * 1e-3) / 1e9,
                     "update": (update_bytes / (update_avg_ms * 1e-3) / 1e9) if opt_kind == "gd" else None},
        "final_loss_head0": float(loss[-1, 0].item()),
        "inner_loss_in_timed_step": bool(args.with_loss),
    }
    if args.offload > 0:
        res["offload"] = offload_bench(tla, inp, Vp, cfg, args, loss_kind, opt_kind)
    if args.conv_fused:
        if cfg.dtype != "bf16" or args.conv_variant != "v3":
            raise SystemExit("--conv-fused takes the bf16 workloads with the 3x3 conv on V")
        res["conv_fused"] = conv_fused_bench(tla, inp, cfg, args, loss_kind, opt_kind, ws, O)
        res["conv_fused"]["split_conv_and_write_ms"] = conv_ms + write_ms
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, cfg, loss=loss_kind, opt=opt_kind,
                                           views_fixed=args.cpu_baseline_views)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

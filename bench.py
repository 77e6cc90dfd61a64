"""Throughput of the silu(group_norm(x)) -> causal conv3d hot path on one MI355X.

A step is one pass of the path over one batch of synthetic input, inputs resident
in HBM. Default workload: the latent-resolution block -- GroupNorm(32)+SiLU fused
into the causal 3x3x3 conv 1024->1024 over [1,4,44,78,1024] bf16 NDHWC with 2
cached frames from a previous pass (gn_silu_stats, then causal_conv3d with the
GroupNorm applied in its operand load, writing y and the new cache).
Other workloads: --config 1..5 (see synthgen/workloads.py).

Prints ONE JSON line. ``value`` = algorithmic conv FLOPs of a step / step time
(TFLOP/s). ``roofline`` is the conv kernel alone (HIP events on the stream it runs
on) against the bf16 dense MFMA peak; ``gn_silu`` is gn_silu_stats + gn_silu_apply on
the same tensor at 6 bytes/element against HBM peak; ``cpu_baseline`` is the fp64
oracle on the host over a bounded sample (rank 0, N=1 only).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import silu_gn_amd as sga  # noqa: E402
import synthgen as sg  # noqa: E402
from synthgen.workloads import WORKLOADS, conv_flops  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 flop/clk (dense)
PEAK_HBM_GBPS = 8000.0
METRIC = "causal conv3d TFLOP/s + GroupNorm+SiLU GB/s (% of MI355X roofline)"


def build_step(wl, dev):
    """Allocate inputs for workload ``wl`` and return (step_fn, conv_only_fn, gn_fns, flops, info)."""
    g, eps = wl.groups, wl.eps
    gamma, beta = wl.gamma(1, dev), wl.beta(1, dev)
    if wl.kind in ("block", "latent"):
        x = wl.x(dev)
        w = wl.conv_weight(1, dev)
        cache = torch.empty((wl.n, 2, wl.h, wl.w, wl.c), dtype=torch.bfloat16, device=dev)
        cache_next = torch.empty_like(cache)
        if wl.cache_from_prev:           # previous pass, untimed: its activated last 2 frames
            xp = wl.x_prev(dev)
            sp = sga.gn_silu_stats(xp, g)
            sga.causal_conv3d(xp, w, None, fuse=(sp, gamma, beta, eps, g), cache_out=cache)
            cin = cache
        else:
            cin = None
        y = torch.empty((wl.n, wl.t, wl.h, wl.w, wl.k), dtype=torch.bfloat16, device=dev)
        stats = torch.empty((wl.n, g, 2), dtype=torch.float64, device=dev)
        ws = torch.empty(sga.gn_silu_stats_workspace(wl.shape, g), dtype=torch.uint8, device=dev)

        def step(timer=None):
            sga.gn_silu_stats(x, g, stats, ws)
            mark(timer, "gn_silu_stats")
            sga.causal_conv3d(x, w, cin, fuse=(stats, gamma, beta, eps, g), y=y, cache_out=cache_next)
            mark(timer, "causal_conv3d (fused)")

        def conv_only():
            sga.causal_conv3d(x, w, cin, fuse=(stats, gamma, beta, eps, g), y=y)

        flops = conv_flops(wl.n, wl.t, wl.h, wl.w, wl.k, wl.c)
        return step, conv_only, (x, stats, ws, gamma, beta), flops, {"conv": "%d->%d 3x3x3 causal" % (wl.c, wl.k)}
    if wl.kind == "upsample":
        x = wl.x(dev)
        wp = sga.upsample2x_prepare_weights(wl.up_weight()).to(dev)
        u = torch.empty((wl.n, wl.t, 2 * wl.h, 2 * wl.w, wl.c), dtype=torch.bfloat16, device=dev)
        w = sg.normal((wl.c, 3, 3, 3, wl.c), wl.seed, sg.W1, std=1 / math.sqrt(27 * wl.c), device=dev)
        y = torch.empty_like(u)
        ushape = tuple(u.shape)
        stats = torch.empty((wl.n, g, 2), dtype=torch.float64, device=dev)
        ws = torch.empty(sga.gn_silu_stats_workspace(ushape, g), dtype=torch.uint8, device=dev)

        def step(timer=None):
            sga.upsample2x_conv_phases(x, wp, y=u)
            mark(timer, "upsample2x_conv_phases")
            sga.gn_silu_stats(u, g, stats, ws)
            mark(timer, "gn_silu_stats")
            sga.causal_conv3d(u, w, None, fuse=(stats, gamma, beta, eps, g), y=y)
            mark(timer, "causal_conv3d (fused)")

        def conv_only():
            sga.causal_conv3d(u, w, None, fuse=(stats, gamma, beta, eps, g), y=y)

        n2, t2, h2, w2, c2 = ushape
        flops = conv_flops(n2, t2, h2, w2, wl.c, c2) + conv_flops(wl.n, wl.t, wl.h, wl.w, wl.c, wl.c, taps=16)
        return step, conv_only, (u, stats, ws, gamma, beta), flops, {"conv": "phases + 512->512 3x3x3 causal"}
    if wl.kind == "resblock":
        x = wl.x(dev)
        params = [(wl.gamma(i, dev), wl.beta(i, dev), wl.conv_weight(i, dev)) for i in (1, 2)]
        caches = [torch.empty((wl.n, 2, wl.h, wl.w, wl.c), dtype=torch.bfloat16, device=dev) for _ in range(4)]
        xp = wl.x_prev(dev)
        h = xp
        for i, (gm, bt, w) in enumerate(params):        # previous pass, untimed
            st = sga.gn_silu_stats(h, g)
            h = sga.causal_conv3d(h, w, None, residual=xp if i == 1 else None, fuse=(st, gm, bt, eps, g),
                                  cache_out=caches[i])
        del h, xp
        hbuf = torch.empty_like(x)
        y = torch.empty_like(x)
        stats = torch.empty((wl.n, g, 2), dtype=torch.float64, device=dev)
        ws = torch.empty(sga.gn_silu_stats_workspace(wl.shape, g), dtype=torch.uint8, device=dev)

        def step(timer=None):
            (g1, b1, w1), (g2, b2, w2) = params
            sga.gn_silu_stats(x, g, stats, ws)
            mark(timer, "gn_silu_stats")
            sga.causal_conv3d(x, w1, caches[0], fuse=(stats, g1, b1, eps, g), y=hbuf, cache_out=caches[2])
            mark(timer, "causal_conv3d (fused)")
            sga.gn_silu_stats(hbuf, g, stats, ws)
            mark(timer, "gn_silu_stats")
            sga.causal_conv3d(hbuf, w2, caches[1], residual=x, fuse=(stats, g2, b2, eps, g), y=y,
                              cache_out=caches[3])
            mark(timer, "causal_conv3d (fused)")

        def conv_only():
            (g1, b1, w1), _ = params
            sga.causal_conv3d(x, w1, caches[0], fuse=(stats, g1, b1, eps, g), y=hbuf)

        flops = 2 * conv_flops(wl.n, wl.t, wl.h, wl.w, wl.c, wl.c)
        return step, conv_only, (x, stats, ws, params[0][0], params[0][1]), flops, {"conv": "2 x 256->256 3x3x3 causal"}
    # head
    x = wl.x(dev)
    w = wl.conv_weight(1, dev)
    video = torch.empty((wl.n, 3, wl.t, 2 * wl.h, 2 * wl.w), dtype=torch.bfloat16, device=dev)
    stats = torch.empty((wl.n, g, 2), dtype=torch.float64, device=dev)
    ws = torch.empty(sga.gn_silu_stats_workspace(wl.shape, g), dtype=torch.uint8, device=dev)

    def step(timer=None):
        sga.gn_silu_stats(x, g, stats, ws)
        mark(timer, "gn_silu_stats")
        sga.head_conv_d2s(x, w, None, None, fuse=(stats, gamma, beta, eps, g), video=video)
        mark(timer, "head_conv_d2s (fused)")

    def conv_only():
        sga.head_conv_d2s(x, w, None, None, fuse=(stats, gamma, beta, eps, g), video=video)

    flops = conv_flops(wl.n, wl.t, wl.h, wl.w, 12, wl.c)
    return step, conv_only, (x, stats, ws, gamma, beta), flops, {"conv": "256->12 3x3x3 causal + d2s"}


def mark(timer, name):
    if timer is not None:
        timer.append((name, torch.cuda.Event(enable_timing=True)))
        timer[-1][1].record()


def time_loop(fn, iters):
    """Average ms of fn() over iters launches, HIP events on the current stream."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def _oracle_cores():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(wl, budget_s=12.0, max_reps=8):
    """The fp64 oracle on the host cores, on the same step as the GPU: GroupNorm statistics
    and activation of all of x, then the causal conv of every output frame with the cache
    (latent / tiny block). The step is repeated until ``budget_s`` seconds have passed
    (at most ``max_reps`` times); value = conv FLOPs of a step / mean step time."""
    import numpy as np
    from oracle import bf16 as obf16
    from oracle import conv as oconv
    from oracle import groupnorm as ogn
    if wl.kind not in ("block", "latent"):
        return None
    xv = wl.x().float().numpy().astype(np.float64)
    gamma, beta = wl.gamma().numpy(), wl.beta().numpy()
    wv = wl.conv_weight().float().numpy().astype(np.float64)
    cache = None
    if wl.cache_from_prev:                       # previous pass, untimed (as on the GPU): its cache
        xp = wl.x_prev().float().numpy().astype(np.float64)      # is its last 2 activated frames
        act, _ = ogn.gn_silu(xp, wl.groups, gamma, beta, wl.eps)
        cache = obf16.decode(obf16.round_rne(act))[:, -2:]
    reps, t0 = 0, time.perf_counter()
    while True:
        act, _ = ogn.gn_silu(xv, wl.groups, gamma, beta, wl.eps)
        oconv.causal_conv3d(obf16.decode(obf16.round_rne(act)), wv, cache)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or reps >= max_reps:
            break
    step_s = dt / reps
    flops = conv_flops(wl.n, wl.t, wl.h, wl.w, wl.k, wl.c)
    return {"value": round(flops / step_s / 1e12, 6), "unit": "TFLOP/s", "cores": int(_oracle_cores()),
            "kind": "oracle",
            "sample": "the whole %s step (GroupNorm+SiLU of all of x, then the causal conv of all %d "
                      "frames with the 2-frame cache), fp64, repeated %d times in %.1f s (%.2f s/step)" %
                      (wl.name, wl.t, reps, dt, step_s)}


def read_traffic(kernel_tag):
    """HBM bytes per launch of the dominant kernel from the committed counter summary, if the
    kernel's sources are unchanged since the counters were taken (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "%s_traffic.txt" % kernel_tag)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for src in fields.get("sources", "").split():
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if not fields.get("sources") or h.hexdigest() != fields.get("sources_sha256"):
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for src in paths:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-pass", action="store_true",
                    help="for hardware-counter runs: one warm-up step, then 5 launches of the dominant "
                         "kernel and 3 plain copies of 1 GiB (the counters' scale), nothing else")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    sga.load_library()
    dev = "cuda:0"
    wl = WORKLOADS[args.config]
    step, conv_only, gn_in, flops, info = build_step(wl, dev)

    if args.profile_pass:
        step()
        torch.cuda.synchronize()
        for _ in range(5):
            conv_only()
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": wl.name, "dominant_launches": 5, "copy_launches": 3,
                          "copy_bytes_read": src.numel() * 2, "copy_bytes_written": dst.numel() * 2}),
              flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timers = []
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        tm = [("start", torch.cuda.Event(enable_timing=True))]
        tm[0][1].record()
        step(tm)
        timers.append(tm)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    stages = {}
    for tm in timers:
        for (_, a), (name, b) in zip(tm[:-1], tm[1:]):
            stages[name] = stages.get(name, 0.0) + a.elapsed_time(b) / args.steps

    # the conv kernel alone (no cache write), and GroupNorm+SiLU unfused on the same tensor
    iters = max(args.steps, 10)
    conv_ms = time_loop(conv_only, iters)
    x, stats, ws, gamma, beta = gn_in
    g = wl.groups
    yb = torch.empty_like(x)
    stats_ms = time_loop(lambda: sga.gn_silu_stats(x, g, stats, ws), iters)
    apply_ms = time_loop(lambda: sga.gn_silu_apply(x, g, stats, gamma, beta, wl.eps, y=yb), iters)
    gn_bytes = 6.0 * x.numel()
    conv_launch_flops = flops if wl.kind != "resblock" else flops / 2
    if wl.kind == "upsample":
        conv_launch_flops = conv_flops(*x.shape[:4], wl.c, wl.c)
    achieved = conv_launch_flops / (conv_ms * 1e-3) / 1e12
    gn_gbps = gn_bytes / ((stats_ms + apply_ms) * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "shape_ndhwc": list(wl.shape), "k": wl.k, "groups": g,
                   "parallelism": "none (1 GPU)", **info},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic("conv_kernel_%s" % wl.name),
                     "kernel": "conv_kernel (causal_conv3d fused)" if wl.kind != "head" else "conv_kernel (head)",
                     "kernel_ms": round(conv_ms, 4)},
        "gn_silu": {"GB/s": round(gn_gbps, 1), "peak": PEAK_HBM_GBPS, "frac": round(gn_gbps / PEAK_HBM_GBPS, 4),
                    "stats_ms": round(stats_ms, 4), "apply_ms": round(apply_ms, 4),
                    "stats_GB/s": round(2.0 * x.numel() / (stats_ms * 1e-3) / 1e9, 1),
                    "apply_GB/s": round(4.0 * x.numel() / (apply_ms * 1e-3) / 1e9, 1),
                    "bytes_per_element": 6},
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

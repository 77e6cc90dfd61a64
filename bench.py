"""Throughput of the silu(group_norm(x)) -> causal conv3d hot path on one MI355X.

A step is one pass of the path over one batch of synthetic input, inputs resident
in HBM. Default workload: the full-resolution residual block over [1,16,352,624,256]
bf16 NDHWC (per-channel mean offsets U(-4,4)), each conv with a 2-frame cache from a
previous pass: gn_silu_stats + gn_silu_apply of x, conv1 (causal_conv3d_next_stats: the
conv, plus norm2's statistics from its epilogue), gn_silu_apply of conv1's output, then
conv2 (causal_conv3d) with the residual x. The convolutions run unfused on the slab
kernel's 256 x 256 tile. Other workloads: --config 1..5 (see synthgen/workloads.py).

Prints ONE JSON line. ``value`` = algorithmic conv FLOPs of a step / step time
(TFLOP/s). ``roofline`` is the conv kernel alone (HIP events on the stream it runs
on) against the bf16 dense MFMA peak, with the HBM traffic and MFMA busy fraction of
the committed rocprofv3 counter summaries when the kernel's sources are unchanged since
they were taken; ``gn_silu`` is gn_silu_stats + gn_silu_apply on the same tensor at 6
bytes/element against HBM peak; ``rms_silu`` is the output head's RMS norm + SiLU on
that tensor at 4 bytes/element; ``other_configs`` is the dominant kernel of every
other workload, launched alone; ``gpu_ceilings`` is what this GPU sustains for those
two resources (libsgnprobe.so: bf16 MFMA with random and with constant operand bits,
HBM streaming read and copy), with each fraction repeated against it;
``cpu_baseline`` is the fp64 oracle on the host over a bounded sample (rank 0, N=1
only).
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


class GnConv:
    """silu(group_norm(src)) -> causal conv on the GPU, with its buffers.

    Unfused (default): gn_silu_stats, gn_silu_apply into ``act``, causal_conv3d on ``act``.
    Fused: gn_silu_stats, then causal_conv3d applying the norm in its operand load.
    ``next_gc``: the conv also emits the statistics of its output for that GnConv
    (causal_conv3d_next_stats), which then skips its own statistics pass (``stats_ready``)."""

    def __init__(self, shape, k, groups, eps, gamma, beta, w, dev, fused, head=False):
        n, t, h, w_, c = shape
        self.g, self.eps, self.gamma, self.beta, self.w = groups, eps, gamma, beta, w
        self.fused, self.head = fused, head
        self.stats = torch.empty((n, groups, 2), dtype=torch.float64, device=dev)
        self.ws = torch.empty(sga.gn_silu_stats_workspace(shape, groups), dtype=torch.uint8, device=dev)
        self.act = None if fused else torch.empty(shape, dtype=torch.bfloat16, device=dev)
        self.shape, self.k = shape, k
        self.nws = None

    def next_ws(self, producer_shape, producer_k):
        """Workspace for a producer conv that emits this GnConv's statistics."""
        if self.nws is None:
            need = sga.causal_conv3d_next_stats_workspace(producer_shape, producer_k, self.g)
            self.nws = torch.empty(max(need, 16), dtype=torch.uint8, device=self.stats.device)
        return self.nws

    def fuse(self):
        return (self.stats, self.gamma, self.beta, self.eps, self.g)

    def __call__(self, src, y, cache_in=None, cache_out=None, residual=None, timer=None, next_gc=None,
                 stats_ready=False):
        if not stats_ready:
            sga.gn_silu_stats(src, self.g, self.stats, self.ws)
            mark(timer, "gn_silu_stats")
        if self.fused:
            a, fuse = src, self.fuse()
        else:
            sga.gn_silu_apply(src, self.g, self.stats, self.gamma, self.beta, self.eps, y=self.act)
            mark(timer, "gn_silu_apply")
            a, fuse = self.act, None
        if self.head:
            sga.head_conv_d2s(a, self.w, cache_in, None, fuse=fuse, video=y, cache_out=cache_out)
            mark(timer, "head_conv_d2s" + (" (fused)" if fuse else ""))
        elif next_gc is not None:
            sga.causal_conv3d_next_stats(a, self.w, next_gc.g, cache_in, residual=residual, fuse=fuse, y=y,
                                         cache_out=cache_out, stats=next_gc.stats,
                                         ws=next_gc.next_ws(self.shape, self.k))
            mark(timer, "causal_conv3d_next_stats" + (" (fused)" if fuse else ""))
        else:
            sga.causal_conv3d(a, self.w, cache_in, residual=residual, fuse=fuse, y=y, cache_out=cache_out)
            mark(timer, "causal_conv3d" + (" (fused)" if fuse else ""))

    def conv_only(self, src, y, cache_in=None, residual=None):
        """The dominant kernel alone: the conv of the step (no cache write)."""
        a, fuse = (src, self.fuse()) if self.fused else (self.act, None)
        if self.head:
            sga.head_conv_d2s(a, self.w, cache_in, None, fuse=fuse, video=y)
        else:
            sga.causal_conv3d(a, self.w, cache_in, residual=residual, fuse=fuse, y=y)


def build_step(wl, dev, fused, separate_stats=False):
    """Allocate inputs for workload ``wl``; return (step, conv_only, gn_inputs, flops, info)."""
    g, eps = wl.groups, wl.eps
    gamma, beta = wl.gamma(1, dev), wl.beta(1, dev)
    conv_name = "causal_conv3d" + (" (fused GroupNorm+SiLU)" if fused else "")
    if wl.kind in ("block", "latent"):
        x = wl.x(dev)
        w = wl.conv_weight(1, dev)
        gc = GnConv(wl.shape, wl.k, g, eps, gamma, beta, w, dev, fused)
        cache = torch.empty((wl.n, 2, wl.h, wl.w, wl.c), dtype=torch.bfloat16, device=dev)
        cache_next = torch.empty_like(cache)
        y = torch.empty((wl.n, wl.t, wl.h, wl.w, wl.k), dtype=torch.bfloat16, device=dev)
        cin = None
        if wl.cache_from_prev:           # previous pass, untimed: its activated last 2 frames
            gc(wl.x_prev(dev), y, None, cache)
            cin = cache

        def step(timer=None):
            gc(x, y, cin, cache_next, timer=timer)

        flops = conv_flops(wl.n, wl.t, wl.h, wl.w, wl.k, wl.c)
        return (step, lambda: gc.conv_only(x, y, cin), (x, gc), flops, flops,
                {"conv": "%d->%d 3x3x3 causal" % (wl.c, wl.k)}, conv_name)
    if wl.kind == "upsample":
        x = wl.x(dev)
        wp = sga.upsample2x_prepare_weights(wl.up_weight()).to(dev)
        ushape = (wl.n, wl.t, 2 * wl.h, 2 * wl.w, wl.c)
        u = torch.empty(ushape, dtype=torch.bfloat16, device=dev)
        w = sg.normal((wl.c, 3, 3, 3, wl.c), wl.seed, sg.W1, std=1 / math.sqrt(27 * wl.c), device=dev)
        gc = GnConv(ushape, wl.c, g, eps, gamma, beta, w, dev, fused)
        y = torch.empty_like(u)
        sga.upsample2x_conv_phases(x, wp, y=u)

        def step(timer=None):
            sga.upsample2x_conv_phases(x, wp, y=u)
            mark(timer, "upsample2x_conv_phases")
            gc(u, y, timer=timer)

        conv = conv_flops(*ushape[:4], wl.c, wl.c)
        flops = conv + conv_flops(wl.n, wl.t, wl.h, wl.w, wl.c, wl.c, taps=16)
        return (step, lambda: gc.conv_only(u, y), (u, gc), flops, conv,
                {"conv": "phases + %d->%d 3x3x3 causal" % (wl.c, wl.c)}, conv_name)
    if wl.kind == "resblock":
        x = wl.x(dev)
        params = [(wl.gamma(i, dev), wl.beta(i, dev), wl.conv_weight(i, dev)) for i in (1, 2)]
        gcs = [GnConv(wl.shape, wl.c, g, eps, gm, bt, w, dev, fused) for gm, bt, w in params]
        caches = [torch.empty((wl.n, 2, wl.h, wl.w, wl.c), dtype=torch.bfloat16, device=dev) for _ in range(4)]
        hbuf = torch.empty_like(x)
        y = torch.empty_like(x)
        xp = wl.x_prev(dev)                                 # previous pass, untimed
        gcs[0](xp, hbuf, None, caches[0])
        gcs[1](hbuf, y, None, caches[1], residual=xp)
        del xp

        def step(timer=None):
            # conv1's epilogue emits norm2's statistics: no statistics pass over h
            nxt = None if separate_stats else gcs[1]
            gcs[0](x, hbuf, caches[0], caches[2], timer=timer, next_gc=nxt)
            gcs[1](hbuf, y, caches[1], caches[3], residual=x, timer=timer, stats_ready=nxt is not None)

        conv = conv_flops(wl.n, wl.t, wl.h, wl.w, wl.c, wl.c)
        return (step, lambda: gcs[0].conv_only(x, hbuf, caches[0]), (x, gcs[0]), 2 * conv, conv,
                {"conv": "2 x %d->%d 3x3x3 causal" % (wl.c, wl.c),
                 "norm2_statistics": "gn_silu_stats over h" if separate_stats
                 else "from conv1's epilogue (causal_conv3d_next_stats)"}, conv_name)
    # head
    x = wl.x(dev)
    w = wl.conv_weight(1, dev)
    gc = GnConv(wl.shape, 12, g, eps, gamma, beta, w, dev, fused, head=True)
    video = torch.empty((wl.n, 3, wl.t, 2 * wl.h, 2 * wl.w), dtype=torch.bfloat16, device=dev)

    def step(timer=None):
        gc(x, video, timer=timer)

    flops = conv_flops(wl.n, wl.t, wl.h, wl.w, 12, wl.c)
    return (step, lambda: gc.conv_only(x, video), (x, gc), flops, flops,
            {"conv": "%d->12 3x3x3 causal + d2s" % wl.c},
            "head_conv_d2s" + (" (fused GroupNorm+SiLU)" if fused else ""))


def up_block_extras(wl, dev, iters):
    """The path's other steps at this workload's shape, each launched alone (HIP events):
    latent: time_upsample_conv (3x1x1 causal conv C -> 2C, halves to frames, steady-state
    pass with a cache); upsample: the phases with the DupUp3D shortcut of a block input of
    x's shape (ft = 1) against the phases alone; full-resolution block: the conv with the
    RMS norm of its output in the epilogue against the conv followed by rms_silu, the conv
    with the RMS norm of its input in the operand load against rms_silu followed by the conv,
    and the conv through Winograd against the direct conv."""
    if wl.kind == "latent":
        x = wl.x(dev)
        wt = sg.normal((2 * wl.c, 3, wl.c), wl.seed, sg.W_TIME, std=1 / math.sqrt(3 * wl.c), device=dev)
        ci = wl.x_prev(dev)[:, -2:].contiguous()
        y = torch.empty((wl.n, 2 * wl.t, wl.h, wl.w, wl.c), dtype=torch.bfloat16, device=dev)
        ms = time_loop(lambda: sga.time_upsample_conv(x, wt, False, ci, y=y), iters)
        fl = 2.0 * wl.n * wl.t * wl.h * wl.w * (2 * wl.c) * 3 * wl.c
        tf = fl / (ms * 1e-3) / 1e12
        return {"time_upsample": {"ms": round(ms, 4), "TFLOP/s": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                                  "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flop_per_launch": fl,
                                  "shape": "x %s -> y [%d,%d,%d,%d,%d] (K = %d)" % (
                                      list(wl.shape), wl.n, 2 * wl.t, wl.h, wl.w, wl.c, 2 * wl.c)}}
    if wl.kind == "upsample":
        x = wl.x(dev)
        src = sg.normal(wl.shape, wl.seed, sg.X_BLOCK, device=dev)
        wp = sga.upsample2x_prepare_weights(wl.up_weight()).to(dev)
        u = torch.empty((wl.n, wl.t, 2 * wl.h, 2 * wl.w, wl.c), dtype=torch.bfloat16, device=dev)
        plain = time_loop(lambda: sga.upsample2x_conv_phases(x, wp, y=u), iters)
        with_sc = time_loop(lambda: sga.upsample2x_conv_phases_shortcut(x, wp, src, 1, False, y=u), iters)
        fl = conv_flops(wl.n, wl.t, wl.h, wl.w, wl.c, wl.c, taps=16)
        return {"upsample_shortcut": {"ms": round(with_sc, 4), "ms_without_shortcut": round(plain, 4),
                                      "TFLOP/s": round(fl / (with_sc * 1e-3) / 1e12, 2),
                                      "shortcut": "DupUp3D of a %s block input, ft = 1" % list(wl.shape)}}
    if wl.kind == "resblock":
        # the decoder's RMS norm of the conv's output: a separate pass (causal_conv3d, then
        # rms_silu) against the norm in the conv's epilogue with y not stored
        x = wl.x(dev)
        w = wl.conv_weight(1, dev)
        gain = wl.gamma(2, dev)
        y = torch.empty_like(x)
        act = torch.empty_like(x)

        def separate():
            sga.causal_conv3d(x, w, y=y)
            sga.rms_silu(y, gain, 1e-6, y=act)
        sep = time_loop(separate, iters)
        epi = time_loop(lambda: sga.causal_conv3d_rms(x, w, gain, 1e-6, act=act, store_y=False), iters)
        out = {"conv_rms_epilogue": {"ms": round(epi, 4), "ms_separate": round(sep, 4),
                                     "form": "causal_conv3d_rms, y not stored (vs causal_conv3d + rms_silu)"}}
        # the RMS norm of the conv's input in its operand load: rms_silu_rstd, then
        # causal_conv3d_rms_input, against rms_silu, then causal_conv3d
        rstd = torch.empty(tuple(x.shape[:4]), dtype=torch.float64, device=dev)

        def separate_in():
            sga.rms_silu(x, gain, 1e-6, y=act)
            sga.causal_conv3d(act, w, y=y)

        def operand_load():
            sga.rms_silu_rstd(x, 1e-6, rstd=rstd)
            sga.causal_conv3d_rms_input(x, w, rstd, gain, y=y)
        sep_in = time_loop(separate_in, iters)
        ol = time_loop(operand_load, iters)
        out["conv_rms_operand_load"] = {"ms": round(ol, 4), "ms_separate": round(sep_in, 4),
                                        "form": "rms_silu_rstd + causal_conv3d_rms_input (vs rms_silu + causal_conv3d)"}
        del rstd
        # the same conv through Winograd F(4x4,3x3) (input transform, 36 component products,
        # output transform) against the direct conv, both on the GroupNorm+SiLU output of x
        st = sga.gn_silu_stats(x, wl.groups)
        sga.gn_silu_apply(x, wl.groups, st, wl.gamma(1, dev), wl.beta(1, dev), wl.eps, y=act)
        u = sga.winograd_prepare_weights(wl.conv_weight(1)).to(dev)
        ws = torch.empty(sga.causal_conv3d_winograd_workspace(wl.shape, wl.c), dtype=torch.uint8, device=dev)
        wino = time_loop(lambda: sga.causal_conv3d_winograd(act, u, y=y, ws=ws), iters)
        direct = time_loop(lambda: sga.causal_conv3d(act, w, y=y), iters)
        fl = conv_flops(wl.n, wl.t, wl.h, wl.w, wl.c, wl.c)
        tiles = ((wl.h + 3) // 4) * ((wl.w + 3) // 4)
        mfl = 36 * 2.0 * wl.n * wl.t * tiles * wl.c * 3 * wl.c
        out["winograd"] = {"ms": round(wino, 4), "ms_direct": round(direct, 4),
                           "TFLOP/s_direct_equivalent": round(fl / (wino * 1e-3) / 1e12, 2),
                           "mfma_flop_per_launch": mfl, "workspace_bytes": ws.numel(),
                           "form": "causal_conv3d_winograd (F(4x4,3x3), bf16 U and V) vs causal_conv3d"}
        del ws
        torch.cuda.empty_cache()
        return out
    return {}


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


def time_each(fn, iters):
    """Per-launch ms of fn() over iters launches (an event pair around each, current stream)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def head_hbm_roofline(n, t, h, w, c, flops):
    """The output head's arithmetic intensity is near the ridge, so its roofline is
    min(MFMA peak, AI x HBM peak): AI = FLOPs / the bytes it must move (x read, video
    written, weights), in FLOP/byte and the TFLOP/s that HBM allows."""
    moved = n * t * h * w * c * 2.0 + n * 3 * t * 4 * h * w * 2.0 + 12 * 27 * c * 2.0
    ai = flops / moved
    hbm_tf = ai * PEAK_HBM_GBPS / 1e3
    return {"ai_flop_per_byte": round(ai, 1), "hbm_bound_TFLOP/s": round(hbm_tf, 1),
            "roofline_TFLOP/s": round(min(PEAK_BF16_TFLOPS, hbm_tf), 1)}


def _oracle_cores():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def _oracle_step(wl, frames):
    """One pass of the workload's step through the fp64 oracle, over the first ``frames``
    frames of its input (the whole input when frames == T); returns a callable."""
    import numpy as np
    from oracle import bf16 as obf16
    from oracle import conv as oconv
    from oracle import groupnorm as ogn

    def f64(t):
        return t.float().numpy().astype(np.float64)

    def rnd(v):
        return obf16.decode(obf16.round_rne(v))

    g, eps = wl.groups, wl.eps
    x = f64(wl.x(frames=frames))
    gamma, beta = wl.gamma().numpy(), wl.beta().numpy()
    if wl.kind in ("block", "latent"):
        w = f64(wl.conv_weight())
        cache = None
        if wl.cache_from_prev:                   # previous pass, untimed (as on the GPU): its cache
            act, _ = ogn.gn_silu(f64(wl.x_prev()), g, gamma, beta, eps)      # is its last 2
            cache = rnd(act)[:, -2:]                                          # activated frames

        def step():
            act, _ = ogn.gn_silu(x, g, gamma, beta, eps)
            oconv.causal_conv3d(rnd(act), w, cache)
        return step
    if wl.kind == "upsample":
        wup = f64(wl.up_weight())
        w = f64(sg.normal((wl.c, 3, 3, 3, wl.c), wl.seed, sg.W1, std=1 / math.sqrt(27 * wl.c)))

        def step():
            u = rnd(oconv.upsample2x_conv(x, wup))
            act, _ = ogn.gn_silu(u, g, gamma, beta, eps)
            oconv.causal_conv3d(rnd(act), w, None)
        return step
    if wl.kind == "resblock":
        (g1, b1, w1), (g2, b2, w2) = [(wl.gamma(i).numpy(), wl.beta(i).numpy(), f64(wl.conv_weight(i)))
                                      for i in (1, 2)]

        def step():
            a1, _ = ogn.gn_silu(x, g, g1, b1, eps)
            h, _ = oconv.causal_conv3d(rnd(a1), w1, None)
            a2, _ = ogn.gn_silu(rnd(h), g, g2, b2, eps)
            oconv.causal_conv3d(rnd(a2), w2, None, residual=x)
        return step
    w = f64(wl.conv_weight())

    def step():
        act, _ = ogn.gn_silu(x, g, gamma, beta, eps)
        oconv.head_conv_d2s(rnd(act), w, None)
    return step


# Frames of each workload's input the CPU baseline runs (about 5-30 s of fp64 work on 16
# host cores); the result is extrapolated linearly to all T frames.
ORACLE_FRAMES = {"tiny_block": 3, "latent_block": 4, "upsample_block": 1, "fullres_resblock": 1,
                 "output_head": 2}


def cpu_baseline(wl, flops, budget_s=12.0, max_reps=8):
    """The fp64 oracle on the host cores, on the workload's step: the whole step for the tiny
    and latent blocks, else the step over its first ORACLE_FRAMES frames, extrapolated
    linearly in the frame count (every stage's work is proportional to the frames it covers).
    The sample is repeated until ``budget_s`` seconds have passed (at most ``max_reps``
    times); value = conv FLOPs of a whole step / extrapolated step time."""
    frames = min(ORACLE_FRAMES[wl.name], wl.t)
    step = _oracle_step(wl, frames)
    reps, t0 = 0, time.perf_counter()
    while True:
        step()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or reps >= max_reps:
            break
    sample_s = dt / reps
    step_s = sample_s * wl.t / frames
    what = ("the whole %s step" % wl.name if frames == wl.t else
            "the %s step over %d of its %d frames (every stage: GroupNorm+SiLU, the convolutions), "
            "extrapolated x%g to all frames" % (wl.name, frames, wl.t, wl.t / frames))
    return {"value": round(flops / step_s / 1e12, 6), "unit": "TFLOP/s", "cores": int(_oracle_cores()),
            "kind": "oracle",
            "sample": "%s, fp64, repeated %d times in %.1f s (%.2f s per sample, %.2f s per step)" %
                      (what, reps, dt, sample_s, step_s)}


def other_configs(index, dev, iters):
    """The dominant kernel of every other workload's step, launched alone after one step
    (HIP events): the conv (unfused, the library's dispatch), the head, and for the upsample
    block also the phases."""
    out = {}
    for i, wl in sorted(WORKLOADS.items()):
        if i == index or wl.kind == "block":
            continue
        step, conv_only, _, _, launch_flops, _, name = build_step(wl, dev, False)
        step()
        ms = time_loop(conv_only, iters)
        tf = launch_flops / (ms * 1e-3) / 1e12
        rec = {"kernel": name, "ms": round(ms, 4), "TFLOP/s": round(tf, 2),
               "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flop_per_launch": launch_flops}
        if wl.kind == "upsample":
            x = wl.x(dev)
            wp = sga.upsample2x_prepare_weights(wl.up_weight()).to(dev)
            u = torch.empty((wl.n, wl.t, 2 * wl.h, 2 * wl.w, wl.c), dtype=torch.bfloat16, device=dev)
            pms = time_loop(lambda: sga.upsample2x_conv_phases(x, wp, y=u), iters)
            pfl = conv_flops(wl.n, wl.t, wl.h, wl.w, wl.c, wl.c, taps=16)
            ptf = pfl / (pms * 1e-3) / 1e12
            rec["phases"] = {"ms": round(pms, 4), "TFLOP/s": round(ptf, 2), "frac": round(ptf / PEAK_BF16_TFLOPS, 4),
                             "flop_per_launch": pfl}
            del x, u
        if wl.kind == "head":
            rec.update(head_hbm_roofline(wl.n, wl.t, wl.h, wl.w, wl.c, launch_flops))
            rec["frac_of_roofline"] = round(tf / rec["roofline_TFLOP/s"], 4)
        out[wl.name] = rec
        del step, conv_only
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def gpu_ceilings(dev):
    """Sustained bf16 MFMA (random / constant operands) and HBM read / copy rates of this GPU,
    from the probe kernels in libsgnprobe.so (about a second in all)."""
    import ctypes
    path = os.path.join(ROOT, "bench_probe", "libsgnprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.sgn_probe_mfma.argtypes = [vp, i32, i32, i32, vp]
    lib.sgn_probe_read.argtypes = [vp, sz, vp, vp]
    lib.sgn_probe_copy.argtypes = [vp, vp, sz, vp]
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    blocks, iters = 512, 8000
    buf = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    flops = 2.0 * 32 * 32 * 16 * 32 * 4 * blocks * iters
    for name, rnd in (("mfma_bf16_random_TFLOP/s", 1), ("mfma_bf16_constant_TFLOP/s", 0)):
        lib.sgn_probe_mfma(buf.data_ptr(), blocks, iters, rnd, stream)
        ms = time_loop(lambda: lib.sgn_probe_mfma(buf.data_ptr(), blocks, iters, rnd, stream), 3)
        out[name] = round(flops / (ms * 1e-3) / 1e12, 1)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    red = torch.empty(2048 * 256 * 16, dtype=torch.uint8, device=dev)
    lib.sgn_probe_read(src.data_ptr(), nbytes, red.data_ptr(), stream)
    ms = time_loop(lambda: lib.sgn_probe_read(src.data_ptr(), nbytes, red.data_ptr(), stream), 10)
    out["hbm_read_GB/s"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    lib.sgn_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream)
    ms = time_loop(lambda: lib.sgn_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream), 10)
    out["hbm_copy_GB/s"] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    del src, dst, red, buf
    torch.cuda.empty_cache()
    return out


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


def read_mfma(kernel_tag):
    """MFMA busy fraction and clock per launch of the dominant kernel from the committed counter
    summary (SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES, GRBM_GUI_ACTIVE), if the kernel's sources
    are unchanged since the counters were taken (else None)."""
    path = os.path.join(ROOT, "profiles", "%s_mfma.txt" % kernel_tag)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    srcs = fields.get("sources", "").split()
    if not srcs or sources_sha256(srcs) != fields.get("sources_sha256"):
        return None
    try:
        return {"mfma_busy": float(fields["mfma_busy"]), "clock_GHz": float(fields["clock_GHz"])}
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
    ap.add_argument("--config", type=int, default=4, choices=sorted(WORKLOADS),
                    help="workload (default 4: the full-resolution residual block, the largest)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the GPU-ceiling probes")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip timing the other workloads' dominant kernels")
    ap.add_argument("--fused", action="store_true",
                    help="apply GroupNorm+SiLU inside the conv's operand load instead of gn_silu_apply")
    ap.add_argument("--separate-stats", action="store_true",
                    help="full-resolution block: take norm2's statistics with gn_silu_stats over h "
                         "instead of from conv1's epilogue")
    ap.add_argument("--profile-pass", action="store_true",
                    help="for hardware-counter runs: one warm-up step, then 5 launches of the dominant "
                         "kernel and 3 plain copies of 1 GiB (the counters' scale), nothing else")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    sga.load_library()
    dev = "cuda:0"
    wl = WORKLOADS[args.config]
    step, conv_only, gn_in, flops, conv_launch_flops, info, conv_name = build_step(wl, dev, args.fused,
                                                                                    args.separate_stats)

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
    # launch-bound workloads: the same step captured once in a HIP graph and replayed (the
    # library's launches are plain stream-ordered kernels, so they capture as they are)
    graph = None
    if wl.kind in ("block", "latent") and not args.fused:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        graph = {"ms_per_step": round(time_loop(g.replay, args.steps), 4), "replays": args.steps,
                 "form": "the step captured in one HIP graph (torch.cuda.graph), replayed"}
        del g

    # the path's other steps at this shape first (so that the conv kernel's last launches
    # are the timed ones below), then the conv kernel alone (no cache write), and
    # GroupNorm+SiLU unfused on the same tensor
    iters = max(args.steps, 10)
    extras = up_block_extras(wl, dev, iters)
    each = sorted(time_each(conv_only, iters))             # per-launch: median and min beside the mean
    conv_ms = time_loop(conv_only, iters)                  # the mean (the kernel trace's last launches)
    x, gc = gn_in
    g = wl.groups
    yb = torch.empty_like(x)
    stats_ms = time_loop(lambda: sga.gn_silu_stats(x, g, gc.stats, gc.ws), iters)
    apply_ms = time_loop(lambda: sga.gn_silu_apply(x, g, gc.stats, gc.gamma, gc.beta, wl.eps, y=yb), iters)
    gn_bytes = 6.0 * x.numel()
    # the output head's norm (RMS norm + SiLU, one read and one write) on the same tensor
    rms_ms = time_loop(lambda: sga.rms_silu(x, gc.gamma, 1e-6, y=yb), iters) if x.shape[-1] % 64 == 0 else None
    achieved = conv_launch_flops / (conv_ms * 1e-3) / 1e12
    gn_gbps = gn_bytes / ((stats_ms + apply_ms) * 1e-3) / 1e9
    flushed = None
    if x.numel() * 2 < (512 << 20):
        # The tensor fits the 256 MB last-level cache: also time each launch after writing
        # 512 MB elsewhere, so that it starts from HBM.
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

        def cold(fn):
            tot = 0.0
            for _ in range(iters):
                scratch.fill_(0)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                torch.cuda.synchronize()
                tot += a.elapsed_time(b)
            return tot / iters

        fs = cold(lambda: sga.gn_silu_stats(x, g, gc.stats, gc.ws))
        fa = cold(lambda: sga.gn_silu_apply(x, g, gc.stats, gc.gamma, gc.beta, wl.eps, y=yb))
        flushed = {"stats_ms": round(fs, 4), "apply_ms": round(fa, 4),
                   "GB/s": round(gn_bytes / ((fs + fa) * 1e-3) / 1e9, 1)}
        del scratch
    ceilings = None if args.no_ceilings else gpu_ceilings(dev)
    # the kernel the dominant launch runs (the library's dispatch rules)
    if wl.kind == "head":
        kname = "head_kernel" if not args.fused and wl.c in (128, 256) else "conv_kernel"
    else:
        kname = "conv_slab_kernel" if not args.fused and wl.k > 128 else "conv_kernel"
    kernel_tag = "%s_%s%s" % (kname, wl.name, "_fused" if args.fused else "")

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
                   "gn_silu": "fused into the conv operand load" if args.fused else "gn_silu_apply, then the conv",
                   "parallelism": "none (1 GPU)", **info},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic(kernel_tag),
                     "kernel": "%s (%s)" % (kernel_tag.split("_" + wl.name)[0], conv_name),
                     "kernel_ms": round(conv_ms, 4), "flop_per_launch": conv_launch_flops,
                     "kernel_ms_median": round(each[len(each) // 2], 4), "kernel_ms_min": round(each[0], 4)},
        "gn_silu": {"GB/s": round(gn_gbps, 1), "peak": PEAK_HBM_GBPS, "frac": round(gn_gbps / PEAK_HBM_GBPS, 4),
                    "stats_ms": round(stats_ms, 4), "apply_ms": round(apply_ms, 4),
                    "stats_GB/s": round(2.0 * x.numel() / (stats_ms * 1e-3) / 1e9, 1),
                    "apply_GB/s": round(4.0 * x.numel() / (apply_ms * 1e-3) / 1e9, 1),
                    "bytes_per_element": 6},
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
    }
    out.update(extras)
    if graph:
        out["graph"] = graph
    if rms_ms:
        rms_gbps = 4.0 * x.numel() / (rms_ms * 1e-3) / 1e9
        out["rms_silu"] = {"GB/s": round(rms_gbps, 1), "peak": PEAK_HBM_GBPS,
                           "frac": round(rms_gbps / PEAK_HBM_GBPS, 4), "ms": round(rms_ms, 4),
                           "bytes_per_element": 4}
    if flushed:
        out["gn_silu"]["cold_cache"] = flushed
    if ceilings:
        out["gpu_ceilings"] = ceilings
        out["roofline"]["frac_of_mfma_random"] = round(achieved / ceilings["mfma_bf16_random_TFLOP/s"], 4)
        # this GPU's rate for this access pattern: the stats' 2 B/element at the read
        # ceiling, the apply's 4 B/element at the copy ceiling
        ceil_s = (2.0 * x.numel() / (ceilings["hbm_read_GB/s"] * 1e9) +
                 4.0 * x.numel() / (ceilings["hbm_copy_GB/s"] * 1e9))
        out["gn_silu"]["ceiling_GB/s"] = round(gn_bytes / ceil_s / 1e9, 1)
        out["gn_silu"]["frac_of_ceiling"] = round(gn_gbps / (gn_bytes / ceil_s / 1e9), 4)
        if rms_ms:
            out["rms_silu"]["frac_of_ceiling"] = round(rms_gbps / ceilings["hbm_copy_GB/s"], 4)
    # HBM bytes per launch of the two GroupNorm kernels from their committed counter summaries
    # (FETCH_SIZE + WRITE_SIZE of the same step's launches), while gn.hip is unchanged
    gs, ga = read_traffic("gn_stats_partial_" + wl.name), read_traffic("gn_apply_kernel_" + wl.name)
    if gs and ga:
        out["gn_silu"]["traffic"] = {"stats_bytes": gs, "apply_bytes": ga,
                                     "bytes_per_element": round((gs + ga) / x.numel(), 3)}
    if wl.kind == "head":
        out["roofline"].update(head_hbm_roofline(wl.n, wl.t, wl.h, wl.w, wl.c, conv_launch_flops))
        out["roofline"]["frac_of_roofline"] = round(achieved / out["roofline"]["roofline_TFLOP/s"], 4)
    mf = read_mfma(kernel_tag)
    if mf:
        out["roofline"].update(mf)
    if not args.no_other_configs:
        out["other_configs"] = other_configs(args.config, dev, iters)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, flops)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

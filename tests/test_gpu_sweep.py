"""Seeded sweeps of small shapes: every entry point on many shape combinations the fixed cases
do not name, against the fp64 oracle. The Winograd form, the phases with the DupUp3D
shortcut and the RMS norm in the operand load run through their fixed-case tests' checks.

Each case draws its shape and options from its own seed, so a failure names a reproducible
case (printed before the launch). The draws cover both kernels of each operation: K above and
below 128 and K % 8 != 0 (the generic tile), one- and multi-tile frames, ragged M and N,
T = 1, two samples, with or without cache, bias and residual.

Gates as in the fixed tests: relative L2 <= 1e-2 and max abs <= 4e-2 against the unrounded
oracle; cache_out bit-exact; the fused GroupNorm form bitwise equal to apply-then-conv; the
conv with the next norm's statistics bitwise equal to the plain conv, its statistics equal
to gn_silu_stats of its output up to fp64 summation order.
"""
import math

import numpy as np
import pytest
import torch

import silu_gn_amd as sga
import synthgen as sg
from oracle import conv as oconv
from oracle import upblock as oup
from tests.helpers import assert_conv_close, bits, vals

pytestmark = pytest.mark.gpu
DEV = "cuda"

CONV_K = [4, 8, 12, 60, 64, 96, 128, 132, 192, 200, 256, 264, 320]
CONV_C = [64, 128, 192, 256]


def _pick(rng, seq):
    return seq[int(rng.integers(0, len(seq)))]


def _conv_case(i):
    rng = np.random.default_rng(7100 + i)
    n = int(rng.integers(1, 3))
    t = int(rng.integers(1, 5))
    h = int(rng.integers(1, 15))
    w = int(rng.integers(1, 41))
    c = _pick(rng, CONV_C)
    k = _pick(rng, CONV_K)
    cache, bias, res, fused = (bool(rng.integers(0, 2)) for _ in range(4))
    return n, t, h, w, c, k, cache, bias, res, fused


@pytest.mark.parametrize("i", range(48))
def test_conv_sweep(i):
    n, t, h, w, c, k, cache, bias, res, fused = _conv_case(i)
    print("case conv sweep", i, (n, t, h, w, c, k), "cache", cache, "bias", bias, "res", res,
          "fused", fused, sga.sgn_conv_plan(sga.SGN_OP_CAUSAL, (n, t, h, w, c), k), flush=True)
    seed = 7100 + i
    a = sg.normal((n, t, h, w, c), seed, sg.X)
    wt = sg.normal((k, 3, 3, 3, c), seed, sg.W1, std=1 / math.sqrt(27 * c))
    ci = sg.normal((n, 2, h, w, c), seed, sg.X_PREV) if cache else None
    b = sg.normal((k,), seed, sg.BETA2, std=0.5, dtype=torch.float32) if bias else None
    r = sg.normal((n, t, h, w, k), seed, sg.GAMMA2) if res else None
    dev = lambda v: v.to(DEV) if v is not None else None   # noqa: E731
    co = torch.empty((n, 2, h, w, c), dtype=torch.bfloat16, device=DEV)
    y = sga.causal_conv3d(dev(a), dev(wt), dev(ci), dev(b), dev(r), cache_out=co)
    # the same conv emitting the next GroupNorm's statistics of y (from the epilogue where
    # K / G allows, else by a statistics pass over y): y bitwise, the statistics against
    # gn_silu_stats(y)
    # (GroupNorm takes K % 8 == 0: 8-channel packets)
    gy = next((g_ for g_ in range(32, 0, -1) if sga.gn_silu_eligible((n, t, h, w, k), g_)), None)
    if gy is not None:
        y_s, st_y = sga.causal_conv3d_next_stats(dev(a), dev(wt), gy, dev(ci), dev(b), dev(r))
        ref_y = sga.gn_silu_stats(y_s, gy)
    if fused:
        # the same conv with GroupNorm+SiLU in its operand load == apply, then the conv
        gamma = sg.normal((c,), seed, sg.GAMMA1, std=0.1, mean=1.0, dtype=torch.float32).to(DEV)
        beta = sg.normal((c,), seed, sg.BETA1, std=0.1, dtype=torch.float32).to(DEV)
        g = 32 if c % 256 == 0 or c in (64, 128) else c // 8   # C / G in {1, 2, 4} or a multiple of 8
        st = sga.gn_silu_stats(dev(a), g)
        act = sga.gn_silu_apply(dev(a), g, st, gamma, beta, 1e-5)
        co_f = torch.empty_like(co)
        co_a = torch.empty_like(co)
        y_f = sga.causal_conv3d(dev(a), dev(wt), dev(ci), dev(b), dev(r), fuse=(st, gamma, beta, 1e-5, g),
                                cache_out=co_f)
        y_a = sga.causal_conv3d(act, dev(wt), dev(ci), dev(b), dev(r), cache_out=co_a)
    torch.cuda.synchronize()
    o, cache_o = oconv.causal_conv3d(vals(a), vals(wt), vals(ci) if cache else None,
                                     b.numpy() if bias else None, vals(r) if res else None)
    assert_conv_close(bits(y), o, "conv sweep %d" % i)
    assert np.array_equal(vals(co), cache_o)
    if gy is not None:
        assert np.array_equal(bits(y_s), bits(y))
        np.testing.assert_allclose(st_y.cpu().numpy(), ref_y.cpu().numpy(), rtol=1e-12, atol=1e-14)
    if fused:
        assert np.array_equal(bits(y_f), bits(y_a))
        assert np.array_equal(bits(co_f), bits(co_a))


@pytest.mark.parametrize("i", range(20))
def test_upsample_sweep(i):
    rng = np.random.default_rng(7300 + i)
    n, t = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    h, w = int(rng.integers(1, 13)), int(rng.integers(1, 25))
    c = _pick(rng, [64, 128, 256])
    k = _pick(rng, [8, 64, 128, 192, 264, 320])
    bias = bool(rng.integers(0, 2))
    print("case upsample sweep", i, (n, t, h, w, c, k), "bias", bias,
          sga.sgn_conv_plan(sga.SGN_OP_PHASES, (n, t, h, w, c), k), flush=True)
    seed = 7300 + i
    x = sg.normal((n, t, h, w, c), seed, sg.X)
    w3 = sg.normal((k, 3, 3, c), seed, sg.W_UP, std=1 / math.sqrt(9 * c))
    b = sg.normal((k,), seed, sg.BETA2, std=0.5, dtype=torch.float32) if bias else None
    wp = sga.upsample2x_prepare_weights(w3).to(DEV)
    y = sga.upsample2x_conv_phases(x.to(DEV), wp, b.to(DEV) if bias else None)
    torch.cuda.synchronize()
    o = oconv.upsample2x_conv(vals(x), vals(w3), b.numpy() if bias else None)
    assert_conv_close(bits(y), o, "upsample sweep %d" % i)


@pytest.mark.parametrize("i", range(16))
def test_head_sweep(i):
    rng = np.random.default_rng(7500 + i)
    n, t = int(rng.integers(1, 3)), int(rng.integers(1, 5))
    h, w = int(rng.integers(1, 13)), int(rng.integers(1, 70))
    c = _pick(rng, [64, 128, 192, 256])                # 128 / 256: the head kernel; else the generic tile
    cache, bias, clamp = (bool(rng.integers(0, 2)) for _ in range(3))
    print("case head sweep", i, (n, t, h, w, c), "cache", cache, "bias", bias, "clamp", clamp, flush=True)
    seed = 7500 + i
    x = sg.normal((n, t, h, w, c), seed, sg.X)
    wt = sg.normal((12, 3, 3, 3, c), seed, sg.W1, std=1 / math.sqrt(27 * c))
    ci = sg.normal((n, 2, h, w, c), seed, sg.X_PREV) if cache else None
    b = sg.normal((12,), seed, sg.BETA2, std=0.5, dtype=torch.float32) if bias else None
    co = torch.empty((n, 2, h, w, c), dtype=torch.bfloat16, device=DEV)
    video = sga.head_conv_d2s(x.to(DEV), wt.to(DEV), ci.to(DEV) if cache else None,
                              b.to(DEV) if bias else None, clamp=clamp, cache_out=co)
    torch.cuda.synchronize()
    ov, oc = oconv.head_conv_d2s(vals(x), vals(wt), vals(ci) if cache else None, b.numpy() if bias else None,
                                 clamp=clamp)
    assert_conv_close(bits(video), ov, "head sweep %d" % i)
    assert np.array_equal(bits(co), bits(torch.from_numpy(oc).to(torch.bfloat16)))


@pytest.mark.parametrize("i", range(16))
def test_time_upsample_sweep(i):
    rng = np.random.default_rng(7700 + i)
    n, t = int(rng.integers(1, 3)), int(rng.integers(1, 5))
    h, w = int(rng.integers(1, 13)), int(rng.integers(1, 30))
    c = _pick(rng, [64, 128, 192, 256])
    first, cache, bias = (bool(rng.integers(0, 2)) for _ in range(3))
    print("case time_upsample sweep", i, (n, t, h, w, c), "first", first, "cache", cache, "bias", bias,
          flush=True)
    seed = 7700 + i
    x = sg.normal((n, t, h, w, c), seed, sg.X)
    wt = sg.normal((2 * c, 3, c), seed, sg.W_TIME, std=1 / math.sqrt(3 * c))
    ci = sg.normal((n, 2, h, w, c), seed, sg.X_PREV) if cache else None
    b = sg.normal((2 * c,), seed, sg.BETA2, std=0.5, dtype=torch.float32) if bias else None
    co = torch.empty((n, 2, h, w, c), dtype=torch.bfloat16, device=DEV)
    y = sga.time_upsample_conv(x.to(DEV), wt.to(DEV), first, ci.to(DEV) if cache else None,
                               b.to(DEV) if bias else None, cache_out=co)
    torch.cuda.synchronize()
    o, oc = oup.time_upsample(vals(x), vals(wt), vals(ci) if cache else None, b.numpy() if bias else None, first)
    yb = bits(y)
    assert yb.shape == o.shape
    start = 1 if first else 0
    if first:
        assert np.array_equal(yb[:, 0], bits(x)[:, 0])
    if o.shape[1] > start:
        assert_conv_close(yb[:, start:], o[:, start:], "time_upsample sweep %d" % i)
    assert np.array_equal(bits(co), bits(torch.from_numpy(oc).to(torch.bfloat16)))


# The entry points with their own fixed-case tests, over drawn shapes through the same checks.
def _bools(rng, m):
    return tuple(bool(rng.integers(0, 2)) for _ in range(m))


@pytest.mark.parametrize("i", range(12))
def test_winograd_sweep(i):
    from tests.test_gpu_winograd import test_winograd_small
    rng = np.random.default_rng(7900 + i)
    n, t = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    h, w = int(rng.integers(1, 15)), int(rng.integers(1, 31))
    c = _pick(rng, [64, 128, 192, 256])
    k = _pick(rng, [136, 192, 256, 264, 320])
    cache, bias, res = _bools(rng, 3)
    test_winograd_small(n, t, h, w, c, k, cache, bias, res)


@pytest.mark.parametrize("i", range(12))
def test_upsample_shortcut_sweep(i):
    from tests.test_gpu_upblock import test_upsample_shortcut_small
    rng = np.random.default_rng(8100 + i)
    n, ts = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    h, w = int(rng.integers(1, 12)), int(rng.integers(1, 24))
    c = _pick(rng, [64, 128])
    k = _pick(rng, [64, 128, 192, 264] if c == 128 else [64, 128, 192, 256, 264])
    cs = k * (1 + int(rng.integers(0, 2)))             # the source has K or 2K channels
    ft = 1 + int(rng.integers(0, 2))
    first, bias = _bools(rng, 2)
    test_upsample_shortcut_small(n, ts, h, w, c, k, cs, ft, first, bias)


@pytest.mark.parametrize("i", range(12))
def test_conv_rms_input_sweep(i):
    from tests.test_gpu_rms import test_conv_rms_input_equals_rms_then_conv
    rng = np.random.default_rng(8300 + i)
    n, t = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    h, w = int(rng.integers(1, 12)), int(rng.integers(1, 30))
    c = _pick(rng, [64, 128, 192, 256])
    k = _pick(rng, [12, 64, 96, 192, 256, 264])
    cache, bias, res = _bools(rng, 3)
    test_conv_rms_input_equals_rms_then_conv(n, t, h, w, c, k, cache, bias, res)

"""Pins of the oracle's convolutions (CPU only).

Against: pure-Python brute force on tiny inputs, PyTorch's float64 conv3d /
conv2d / interpolate / pixel_shuffle as independent library routines, closed
forms (delta and all-ones kernels), causality, pass splitting, and the
nearest-x2 == four-phase identity (tap table from the binding.cpp page).
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import conv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def _rand(*shape):
    return rng.standard_normal(shape)


def _brute_causal(a, w, cache, bias, residual):
    n, t, h, wd, c = a.shape
    k = w.shape[0]
    out = np.zeros((n, t, h, wd, k))
    for ni, ti, hi, wi, ki in itertools.product(range(n), range(t), range(h), range(wd), range(k)):
        s = 0.0
        for dt, dh, dw, ci in itertools.product(range(3), range(3), range(3), range(c)):
            tt, hh, ww = ti + dt - 2, hi + dh - 1, wi + dw - 1
            if not (0 <= hh < h and 0 <= ww < wd):
                continue
            v = a[ni, tt, hh, ww, ci] if tt >= 0 else (cache[ni, tt + 2, hh, ww, ci] if cache is not None else 0.0)
            s += w[ki, dt, dh, dw, ci] * v
        out[ni, ti, hi, wi, ki] = s + (bias[ki] if bias is not None else 0) + (
            residual[ni, ti, hi, wi, ki] if residual is not None else 0)
    return out


@pytest.mark.parametrize("t", [1, 2, 3])
@pytest.mark.parametrize("with_cache", [False, True])
def test_causal_conv_brute_force(t, with_cache):
    a = _rand(1, t, 3, 4, 2)
    w = _rand(3, 3, 3, 3, 2)
    cache = _rand(1, 2, 3, 4, 2) if with_cache else None
    bias = np.float32([0.5, -1.0, 0.25])
    res = _rand(1, t, 3, 4, 3)
    out, cache_out = conv.causal_conv3d(a, w, cache, bias, res)
    want = _brute_causal(a, w, cache, bias.astype(np.float64), res)
    assert np.allclose(out, want, rtol=1e-13, atol=1e-13)
    p = np.concatenate([cache if with_cache else np.zeros((1, 2, 3, 4, 2)), a], axis=1)
    assert np.array_equal(cache_out, p[:, -2:])


def test_causal_conv_vs_torch_conv3d():
    n, t, h, w, c, k = 2, 4, 7, 9, 8, 5
    a, wt, cache = _rand(n, t, h, w, c), _rand(k, 3, 3, 3, c), _rand(n, 2, h, w, c)
    out, _ = conv.causal_conv3d(a, wt, cache)
    p = torch.from_numpy(np.concatenate([cache, a], axis=1)).permute(0, 4, 1, 2, 3)
    ref = F.conv3d(p, torch.from_numpy(wt).permute(0, 4, 1, 2, 3), padding=(0, 1, 1))
    assert np.allclose(out, ref.permute(0, 2, 3, 4, 1).numpy(), rtol=1e-12, atol=1e-12)


def test_delta_kernels():
    a, cache = _rand(1, 3, 4, 5, 4), _rand(1, 2, 4, 5, 4)
    w = np.zeros((4, 3, 3, 3, 4))
    for ki in range(4):
        w[ki, 2, 1, 1, ki] = 1.0                 # centre tap of the newest frame
    out, _ = conv.causal_conv3d(a, w, cache)
    assert np.array_equal(out, a)
    w0 = np.zeros((4, 3, 3, 3, 4))
    for ki in range(4):
        w0[ki, 0, 1, 1, ki] = 1.0                # oldest frame: out[t] = P[t]
    out0, _ = conv.causal_conv3d(a, w0, cache)
    p = np.concatenate([cache, a], axis=1)
    assert np.array_equal(out0, p[:, :3])


def test_all_ones_constant_input():
    c, v = 4, 0.5
    a = np.full((1, 3, 4, 5, c), v)
    w = np.ones((1, 3, 3, 3, c))
    out, _ = conv.causal_conv3d(a, w, np.full((1, 2, 4, 5, c), v))
    o = out[0, :, :, :, 0] / (c * v)
    assert np.all(o[:, 1:-1, 1:-1] == 27) and np.all(o[:, 0, 1:-1] == 18) and np.all(o[:, 0, 0] == 12)
    outz, _ = conv.causal_conv3d(a, w, None)
    oz = outz[0, :, :, :, 0] / (c * v)
    assert oz[0, 2, 2] == 9 and oz[0, 0, 2] == 6 and oz[0, 0, 0] == 4
    assert oz[1, 2, 2] == 18 and oz[1, 0, 2] == 12 and oz[1, 0, 0] == 8
    assert oz[2, 2, 2] == 27


def test_causality():
    a, w, cache = _rand(1, 5, 4, 4, 3), _rand(2, 3, 3, 3, 3), _rand(1, 2, 4, 4, 3)
    base, _ = conv.causal_conv3d(a, w, cache)
    for t0 in range(5):
        b = a.copy()
        b[0, t0] += 1.0
        pert, _ = conv.causal_conv3d(b, w, cache)
        assert np.array_equal(pert[:, :t0], base[:, :t0])
        for tt in range(t0, min(5, t0 + 3)):
            assert not np.allclose(pert[:, tt], base[:, tt])
        if t0 + 3 < 5:
            assert np.array_equal(pert[:, t0 + 3:], base[:, t0 + 3:])


@pytest.mark.parametrize("t1", [1, 2, 3])
def test_pass_split(t1):
    a, w, c0 = _rand(1, 5, 3, 4, 3), _rand(2, 3, 3, 3, 3), _rand(1, 2, 3, 4, 3)
    whole, cache_whole = conv.causal_conv3d(a, w, c0)
    first, c1 = conv.causal_conv3d(a[:, :t1], w, c0)
    second, c2 = conv.causal_conv3d(a[:, t1:], w, c1)
    assert np.allclose(np.concatenate([first, second], axis=1), whole, rtol=1e-14, atol=1e-14)
    assert np.array_equal(c2, cache_whole)


def test_sampled_patches_match_full():
    a, w, cache = _rand(1, 3, 5, 6, 4), _rand(3, 3, 3, 3, 4), _rand(1, 2, 5, 6, 4)
    full, _ = conv.causal_conv3d(a, w, cache)
    pos = np.array(list(itertools.product([0], range(3), range(5), range(6))))
    got = conv.conv_at(conv.causal_patches(a, cache, pos), w)
    assert np.allclose(got, full.reshape(-1, 3), rtol=1e-13, atol=1e-13)
    # with an activation applied to the current frames only
    act = lambda v, n: np.tanh(v)          # noqa: E731
    full2, _ = conv.causal_conv3d(np.tanh(a), w, cache)
    got2 = conv.conv_at(conv.causal_patches(a, cache, pos, act=act), w)
    assert np.allclose(got2, full2.reshape(-1, 3), rtol=1e-13, atol=1e-13)


def test_phase_tap_table_matches_pages_rule():
    table = json.load(open(os.path.join(GOLDEN, "phase_taps.json")))["rows_for_phase"]
    w = np.zeros((1, 3, 3, 1))
    for a in (0, 1):
        for r in range(3):
            w[:] = 0
            w[0, r, 1, 0] = 1.0
            pw = conv.phase_weights(w)            # [a, b, k, u, v, c]
            u = [uu for uu in (0, 1) if pw[a, 1, 0, uu, :, 0].sum() != 0]
            assert len(u) == 1
            assert r in table[str(a)]["u%d" % u[0]]


def test_upsample_direct_vs_torch():
    x, w = _rand(1, 2, 5, 7, 6), _rand(4, 3, 3, 6)
    out = conv.upsample2x_conv(x, w)
    xt = torch.from_numpy(x[0]).permute(0, 3, 1, 2)                    # T, C, H, W
    up = F.interpolate(xt, scale_factor=2, mode="nearest")
    ref = F.conv2d(up, torch.from_numpy(w).permute(0, 3, 1, 2), padding=1)
    assert np.allclose(out[0], ref.permute(0, 2, 3, 1).numpy(), rtol=1e-12, atol=1e-12)


def test_phase_identity():
    x, w = _rand(1, 3, 5, 7, 6), _rand(4, 3, 3, 6)
    direct = conv.upsample2x_conv(x, w)
    phases = conv.upsample2x_conv_phases(x, conv.phase_weights(w))
    assert np.allclose(phases, direct, rtol=1e-12, atol=1e-12)


def test_upsample_sampled_matches_full():
    x, w = _rand(1, 2, 4, 5, 3), _rand(2, 3, 3, 3)
    full = conv.upsample2x_conv(x, w)
    pos = np.array(list(itertools.product([0], range(2), range(8), range(10))))
    got = conv.upsample2x_conv_at(x, w, pos)
    assert np.allclose(got, full.reshape(-1, 2), rtol=1e-13, atol=1e-13)


def test_depth_to_space_matches_pixel_shuffle_and_inverts():
    y = _rand(1, 2, 3, 4, 12)
    v = conv.depth_to_space(y)
    yt = torch.from_numpy(y[0]).permute(0, 3, 1, 2)                    # T, 12, H, W
    ref = F.pixel_shuffle(yt, 2).permute(1, 0, 2, 3).numpy()            # 3, T, 2H, 2W
    assert np.array_equal(v[0], ref)
    back = F.pixel_unshuffle(torch.from_numpy(v[0]).permute(1, 0, 2, 3), 2).permute(0, 2, 3, 1).numpy()
    assert np.array_equal(back, y[0])
    assert v.size == y.size


def test_head_is_conv_then_d2s_then_clamp():
    a, w, cache = _rand(1, 2, 3, 4, 8), _rand(12, 3, 3, 3, 8), _rand(1, 2, 3, 4, 8)
    bias = np.float32(np.linspace(-1, 1, 12))
    video, cache_out = conv.head_conv_d2s(a, w, cache, bias, clamp=True)
    out, _ = conv.causal_conv3d(a, w, cache, bias)
    assert np.array_equal(video, np.clip(conv.depth_to_space(out), -1, 1))
    assert np.array_equal(cache_out, a[:, -2:])

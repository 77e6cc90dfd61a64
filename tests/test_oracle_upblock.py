"""Pins of the oracle's up-block steps (CPU only): the temporal x2 and the DupUp3D shortcut.

Against: pure-Python brute force on tiny inputs, PyTorch's float64 conv3d followed by the
channel-halves-to-frames interleave, closed forms (a pass-through kernel), causality and
pass splitting for the time conv; PyTorch's nearest interpolate (channel count kept) and
pixel_shuffle (no channel repeat) for DupUp3D, and the first-pass frame drop.
"""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import upblock

rng = np.random.default_rng(4321)


def _rand(*shape):
    return rng.standard_normal(shape)


def _brute_time(x, w, cache, bias, first):
    n, t, h, wd, c = x.shape
    start = 1 if first else 0
    nf = t - start
    out = np.zeros((n, start + 2 * nf, h, wd, c))
    for ni, f, hi, wi, ci in itertools.product(range(n), range(start + 2 * nf), range(h), range(wd), range(c)):
        if first and f == 0:
            out[ni, f, hi, wi, ci] = x[ni, 0, hi, wi, ci]
            continue
        i, s = divmod(f - start, 2)
        k = s * c + ci
        acc = bias[k] if bias is not None else 0.0
        for dt, cc in itertools.product(range(3), range(c)):
            j = i + dt - 2
            v = x[ni, start + j, hi, wi, cc] if j >= 0 else (cache[ni, j + 2, hi, wi, cc] if cache is not None else 0.0)
            acc += w[k, dt, cc] * v
        out[ni, f, hi, wi, ci] = acc
    return out


@pytest.mark.parametrize("t,first", [(1, False), (3, False), (1, True), (2, True), (4, True)])
@pytest.mark.parametrize("with_cache", [False, True])
def test_time_upsample_brute_force(t, first, with_cache):
    x = _rand(2, t, 2, 3, 2)
    w = _rand(4, 3, 2)
    cache = _rand(2, 2, 2, 3, 2) if with_cache else None
    bias = np.float32([0.5, -1.0, 0.25, 2.0])
    out, cache_out = upblock.time_upsample(x, w, cache, bias, first)
    assert out.shape == (2, (1 if first else 0) + 2 * (t - (1 if first else 0)), 2, 3, 2)
    assert np.allclose(out, _brute_time(x, w, cache, bias.astype(np.float64), first), rtol=1e-13, atol=1e-13)
    p = np.concatenate([cache if with_cache else np.zeros((2, 2, 2, 3, 2)), x[:, 1 if first else 0:]], axis=1)
    assert np.array_equal(cache_out, p[:, -2:])


@pytest.mark.parametrize("first", [False, True])
def test_time_upsample_vs_torch_conv3d(first):
    n, t, h, w, c = 2, 5, 4, 6, 8
    x = _rand(n, t, h, w, c)
    wt = _rand(2 * c, 3, c)
    cache = _rand(n, 2, h, w, c)
    bias = rng.standard_normal(2 * c).astype(np.float32)
    out, _ = upblock.time_upsample(x, wt, cache, bias, first)
    start = 1 if first else 0
    p = torch.from_numpy(np.concatenate([cache, x[:, start:]], axis=1)).permute(0, 4, 1, 2, 3)   # N C T H W
    ker = torch.from_numpy(wt).permute(0, 2, 1)[..., None, None]                                # 2C, C, 3, 1, 1
    y = F.conv3d(p, ker, torch.from_numpy(bias.astype(np.float64)))                             # N, 2C, nf, H, W
    nf = t - start
    y = torch.stack((y[:, :c], y[:, c:]), dim=3).reshape(n, c, 2 * nf, h, w)                    # frames 2i, 2i + 1
    want = y.permute(0, 2, 3, 4, 1).numpy()
    if first:
        want = np.concatenate([x[:, :1], want], axis=1)
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)


def test_time_upsample_pass_through_kernel():
    # w[s C + c, 2, c] = 1: every frame of x (after the first) appears twice, plus the bias
    n, t, h, w, c = 1, 4, 3, 5, 4
    x = _rand(n, t, h, w, c)
    wt = np.zeros((2 * c, 3, c))
    for s in range(2):
        wt[s * c + np.arange(c), 2, np.arange(c)] = 1.0
    bias = np.float32(np.arange(2 * c) * 0.5)
    out, _ = upblock.time_upsample(x, wt, _rand(n, 2, h, w, c), bias, first=True)
    assert np.array_equal(out[:, 0], x[:, 0])
    for j in range(1, t):
        assert np.allclose(out[:, 2 * j - 1], x[:, j] + bias[:c], atol=1e-15)
        assert np.allclose(out[:, 2 * j], x[:, j] + bias[c:], atol=1e-15)


def test_time_upsample_causal_and_pass_split():
    n, t, h, w, c = 1, 6, 2, 3, 4
    x = _rand(n, t, h, w, c)
    wt = _rand(2 * c, 3, c)
    bias = rng.standard_normal(2 * c).astype(np.float32)
    whole, cache_whole = upblock.time_upsample(x, wt, None, bias, first=True)
    # causality: a change in x frame j >= 1 leaves output frames before 2j - 1 alone
    x2 = x.copy()
    x2[:, 3] += 1.0
    moved, _ = upblock.time_upsample(x2, wt, None, bias, first=True)
    assert np.array_equal(moved[:, :5], whole[:, :5]) and not np.allclose(moved[:, 5], whole[:, 5])
    # two passes carrying the cache give the frames of one pass
    a, ca = upblock.time_upsample(x[:, :2], wt, None, bias, first=True)
    b, cb = upblock.time_upsample(x[:, 2:], wt, ca, bias, first=False)
    assert np.allclose(np.concatenate([a, b], axis=1), whole, rtol=1e-13, atol=1e-13)
    assert np.array_equal(cb, cache_whole)


def test_time_upsample_at_matches():
    n, t, h, w, c = 2, 4, 3, 4, 8
    x = _rand(n, t, h, w, c)
    wt = _rand(2 * c, 3, c)
    cache = _rand(n, 2, h, w, c)
    bias = rng.standard_normal(2 * c).astype(np.float32)
    for first in (False, True):
        out, _ = upblock.time_upsample(x, wt, cache, bias, first)
        pos = np.array(list(itertools.product(range(n), range(out.shape[1]), range(h), range(w))))
        got = upblock.time_upsample_at(x, wt, cache, bias, first, pos)
        assert np.allclose(got, out[pos[:, 0], pos[:, 1], pos[:, 2], pos[:, 3]], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("first", [False, True])
def test_dup_up3d_same_channels_is_nearest(first):
    # Cin = Cout, ft = fs = 2: rep = 8 copies of each channel cover (a, b, d), i.e. nearest x2
    x = _rand(2, 3, 4, 5, 6)
    out = upblock.dup_up3d(x, 6, 2, 2, first)
    want = F.interpolate(torch.from_numpy(x).permute(0, 4, 1, 2, 3), scale_factor=2, mode="nearest")
    want = want.permute(0, 2, 3, 4, 1).numpy()
    assert np.array_equal(out, want[:, 1:] if first else want)


def test_dup_up3d_no_repeat_is_pixel_shuffle():
    # Cin = Cout fs^2, ft = 1: rep = 1, channel (c, b, d) goes to (fs h + b, fs w + d)
    x = _rand(2, 3, 4, 5, 12)
    out = upblock.dup_up3d(x, 3, 1, 2)
    for t in range(3):
        want = F.pixel_shuffle(torch.from_numpy(x[:, t]).permute(0, 3, 1, 2), 2).permute(0, 2, 3, 1).numpy()
        assert np.array_equal(out[:, t], want)


def _brute_dup(x, cout, ft, fs, first):
    n, t, h, w, cin = x.shape
    rep = cout * ft * fs * fs // cin
    drop = ft - 1 if first else 0
    out = np.zeros((n, t * ft - drop, h * fs, w * fs, cout))
    for ni, f, y, xx, c in itertools.product(*(range(s) for s in out.shape)):
        tt, a = divmod(f + drop, ft)
        hh, b = divmod(y, fs)
        ww, d = divmod(xx, fs)
        out[ni, f, y, xx, c] = x[ni, tt, hh, ww, (((c * ft + a) * fs + b) * fs + d) // rep]
    return out


@pytest.mark.parametrize("cin,cout,ft,fs", [(4, 4, 2, 2), (4, 2, 1, 2), (8, 4, 2, 2), (2, 4, 2, 2), (3, 6, 2, 1)])
@pytest.mark.parametrize("first", [False, True])
def test_dup_up3d_brute_force_and_sampled(cin, cout, ft, fs, first):
    x = _rand(1, 3, 2, 3, cin)
    out = upblock.dup_up3d(x, cout, ft, fs, first)
    assert np.array_equal(out, _brute_dup(x, cout, ft, fs, first))
    pos = np.array(list(itertools.product(range(1), range(out.shape[1]), range(out.shape[2]), range(out.shape[3]))))
    got = upblock.dup_up3d_at(x, cout, ft, fs, first, pos)
    assert np.array_equal(got, out[pos[:, 0], pos[:, 1], pos[:, 2], pos[:, 3]])

"""Convolutions of the decoder path, plain definitions in float64 (test infrastructure only).

Pages: FastVideo ``wan22_vae_decode/solution/binding.cpp`` --
* Decoder::conv: a causal convolution pads kt - 1 = 2 frames in front, taken
  from the per-conv cache (zeros before the first pass), pads the spatial dims
  by kh/2 = kw/2 = 1 with zeros, and afterwards keeps the last 2 frames of the
  padded input as the new cache;
* prepare(): nearest-x2 followed by a 3x3 convolution equals four 2x2
  convolutions at the low resolution, one per output phase (a, b);
* Decoder::output_head: the 3x3x3 head convolution to 12 channels, whose
  channels are unfolded 2x2 into the RGB video.

Layouts: activations (N, T, H, W, C); 3-D weights (K, 3, 3, 3, C) with taps
ordered (dt, dh, dw) and dt = 0 multiplying the oldest frame t - 2; 2-D
weights (K, 3, 3, C). All arithmetic is float64 on exact bf16 / fp32 inputs.
"""
from __future__ import annotations

import numpy as np


def causal_input(a, cache=None):
    """P = cat(cache, a) along time, (N, T + 2, H, W, C); a missing cache is zeros."""
    a = np.asarray(a, dtype=np.float64)
    n, t, h, w, c = a.shape
    if cache is None:
        cache = np.zeros((n, 2, h, w, c))
    cache = np.asarray(cache, dtype=np.float64)
    assert cache.shape == (n, 2, h, w, c)
    return np.concatenate([cache, a], axis=1)


def causal_conv3d(a, weight, cache=None, bias=None, residual=None):
    """Causal 3x3x3 convolution.

    out[n,t,h,w,k] = bias[k] + residual[n,t,h,w,k]
        + sum_{dt,dh,dw in 0..2} sum_c weight[k,dt,dh,dw,c] * P[n, t+dt, h+dh-1, w+dw-1, c]
    with P = cat(cache, a) and P = 0 outside the spatial range.
    Returns (out float64 (N, T, H, W, K), cache_out = P[:, T:T+2]).
    """
    p = causal_input(a, cache)
    n, t2, h, w, c = p.shape
    t = t2 - 2
    wt = np.asarray(weight, dtype=np.float64)
    k = wt.shape[0]
    assert wt.shape == (k, 3, 3, 3, c)
    pp = np.pad(p, ((0, 0), (0, 0), (1, 1), (1, 1), (0, 0)))
    out = np.zeros((n, t, h, w, k))
    for dt in range(3):
        for dh in range(3):
            for dw in range(3):
                window = pp[:, dt:dt + t, dh:dh + h, dw:dw + w, :].reshape(-1, c)
                out += (window @ wt[:, dt, dh, dw, :].T).reshape(n, t, h, w, k)
    if bias is not None:
        out += np.asarray(bias, np.float32).astype(np.float64)
    if residual is not None:
        out += np.asarray(residual, dtype=np.float64)
    return out, p[:, t:t + 2].copy()


def causal_patches(source, cache, positions, act=None):
    """The 3x3x3 input patches of chosen output positions, (S, 3, 3, 3, C) float64.

    ``positions`` is an (S, 4) integer array of (n, t, h, w). Frame t + dt - 2
    comes from ``source`` when >= 0 (passed through ``act`` if given: the
    activation of a fused normalisation, applied to each gathered value with its
    sample index) and from ``cache`` (already activated; zeros if None)
    otherwise; spatial neighbours outside the frame are zero.
    """
    pos = np.asarray(positions, dtype=np.int64)
    n_, t_, h_, w_ = (pos[:, i] for i in range(4))
    _, _, hh_max, ww_max, c = source.shape
    s = pos.shape[0]
    out = np.zeros((s, 3, 3, 3, c))
    for dt in range(3):
        tt = t_ + dt - 2
        for dh in range(3):
            hh = h_ + dh - 1
            for dw in range(3):
                ww = w_ + dw - 1
                inside = (hh >= 0) & (hh < hh_max) & (ww >= 0) & (ww < ww_max)
                cur = inside & (tt >= 0)
                if cur.any():
                    vals = np.asarray(source[n_[cur], tt[cur], hh[cur], ww[cur]], dtype=np.float64)
                    if act is not None:
                        vals = act(vals, n_[cur])
                    out[cur, dt, dh, dw] = vals
                old = inside & (tt < 0)
                if cache is not None and old.any():
                    out[old, dt, dh, dw] = np.asarray(
                        cache[n_[old], tt[old] + 2, hh[old], ww[old]], dtype=np.float64)
    return out


def conv_at(patches, weight, bias=None):
    """Outputs at sampled positions from their patches: (S, 27C) @ (27C, K), float64."""
    s = patches.shape[0]
    wt = np.asarray(weight, dtype=np.float64)
    k = wt.shape[0]
    out = patches.reshape(s, -1) @ wt.reshape(k, -1).T
    if bias is not None:
        out = out + np.asarray(bias, np.float32).astype(np.float64)
    return out


def nearest_up2(x):
    """Nearest-neighbour x2 in H and W: up[.., Y, X, :] = x[.., Y // 2, X // 2, :]."""
    x = np.asarray(x, dtype=np.float64)
    return np.repeat(np.repeat(x, 2, axis=2), 2, axis=3)


def conv2d_same(x, weight, bias=None):
    """Per-frame 3x3 convolution with 1-pixel zero padding, x (N, T, H, W, C), weight (K, 3, 3, C)."""
    x = np.asarray(x, dtype=np.float64)
    n, t, h, w, c = x.shape
    wt = np.asarray(weight, dtype=np.float64)
    k = wt.shape[0]
    xp = np.pad(x, ((0, 0), (0, 0), (1, 1), (1, 1), (0, 0)))
    out = np.zeros((n, t, h, w, k))
    for r in range(3):
        for s in range(3):
            out += (xp[:, :, r:r + h, s:s + w, :].reshape(-1, c) @ wt[:, r, s, :].T).reshape(n, t, h, w, k)
    if bias is not None:
        out += np.asarray(bias, np.float32).astype(np.float64)
    return out


def upsample2x_conv(x, weight, bias=None):
    """The definition: nearest-x2, then a 3x3 'same' convolution on the 2H x 2W grid."""
    return conv2d_same(nearest_up2(x), weight, bias)


def upsample2x_conv_at(x, weight, positions):
    """Outputs of the direct form at sampled high-resolution positions (n, t, Y, X), (S, K)."""
    x = np.asarray(x)
    pos = np.asarray(positions, dtype=np.int64)
    _, _, h, w, c = x.shape
    s = pos.shape[0]
    patches = np.zeros((s, 3, 3, c))
    for r in range(3):
        yy = pos[:, 2] + r - 1
        for q in range(3):
            xx = pos[:, 3] + q - 1
            inside = (yy >= 0) & (yy < 2 * h) & (xx >= 0) & (xx < 2 * w)
            patches[inside, r, q] = x[pos[inside, 0], pos[inside, 1], yy[inside] // 2, xx[inside] // 2]
    wt = np.asarray(weight, dtype=np.float64)
    return patches.reshape(s, -1) @ wt.reshape(wt.shape[0], -1).T


def phase_weights(weight):
    """The four 2x2 phase kernels of a 3x3 kernel, float64, (2, 2, K, 2, 2, C) indexed [a, b, k, u, v, c].

    Output pixel (2i + a, 2j + b) of nearest-x2 + 3x3 reads up-grid row 2i + a + r - 1,
    i.e. low-res row floor((a + r - 1) / 2) + i; tap r joins phase tap u when that
    row is i + u + a - 1 (binding.cpp, prepare(); same for columns with b, s, v).
    """
    wt = np.asarray(weight, dtype=np.float64)
    k, _, _, c = wt.shape
    out = np.zeros((2, 2, k, 2, 2, c))
    for a in range(2):
        for b in range(2):
            for r in range(3):
                u = (a + r - 1) // 2 - a + 1
                for s in range(3):
                    v = (b + s - 1) // 2 - b + 1
                    out[a, b, :, u, v, :] += wt[:, r, s, :]
    return out


def upsample2x_conv_phases(x, pw, bias=None):
    """The phase form: out[n,t,2i+a,2j+b,k] = sum_{u,v,c} pw[a,b,k,u,v,c] * x[n,t,i+u+a-1,j+v+b-1,c]."""
    x = np.asarray(x, dtype=np.float64)
    n, t, h, w, c = x.shape
    k = pw.shape[2]
    xp = np.pad(x, ((0, 0), (0, 0), (1, 1), (1, 1), (0, 0)))
    out = np.zeros((n, t, 2 * h, 2 * w, k))
    for a in range(2):
        for b in range(2):
            acc = np.zeros((n, t, h, w, k))
            for u in range(2):
                for v in range(2):
                    win = xp[:, :, u + a:u + a + h, v + b:v + b + w, :].reshape(-1, c)
                    acc += (win @ pw[a, b, :, u, v, :].T).reshape(n, t, h, w, k)
            out[:, :, a::2, b::2, :] = acc
    if bias is not None:
        out += np.asarray(bias, np.float32).astype(np.float64)
    return out


def depth_to_space(y):
    """(N, T, H, W, 12) -> video (N, 3, T, 2H, 2W) with video[n,c,t,2h+dy,2w+dx] = y[n,t,h,w,4c+2dy+dx]."""
    y = np.asarray(y)
    n, t, h, w, k = y.shape
    assert k == 12
    v = y.reshape(n, t, h, w, 3, 2, 2)            # [.., c, dy, dx]
    v = v.transpose(0, 4, 1, 2, 5, 3, 6)           # n, c, t, h, dy, w, dx
    return v.reshape(n, 3, t, 2 * h, 2 * w)


def head_conv_d2s(a, weight, cache=None, bias=None, clamp=False):
    """Output head: causal 3x3x3 conv to 12 channels, 2x2 depth-to-space, optional clamp to [-1, 1].

    Returns (video float64 (N, 3, T, 2H, 2W), cache_out).
    """
    out, cache_out = causal_conv3d(a, weight, cache, bias)
    video = depth_to_space(out)
    if clamp:
        video = np.clip(video, -1.0, 1.0)
    return video, cache_out

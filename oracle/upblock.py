"""The rest of an up block: temporal x2 and the DupUp3D shortcut, plain float64 definitions
(test infrastructure only).

Pages: FastVideo ``wan22_vae_decode/solution/binding.cpp`` --
* Decoder::up_block (the seam after the three resnets of blocks 0 and 1): the causal
  3x1x1 time convolution runs on the block's frames after the first one when this is the
  video's first pass (that frame goes straight to the output), with its own 2-frame cache in
  front and no normalisation (copy-only norm_pad), and writes a frame-interleaved tensor:
  every input frame becomes two output frames (time_upsample);
* the same function, after the four phase convolutions: one pass interleaves the phases and
  adds the bias and the DupUp3D shortcut of the block's input (resample_upsample).

Readings (the pages print neither formula):
* time conv: weight (2C, 3, C), tap dt = 0 on the oldest frame; output frame first + 2i + s
  holds channels s*C .. s*C + C - 1 of the conv's frame i (the first half is the earlier
  frame);
* DupUp3D(Cin -> Cout, factor ft in time, fs in space): every input channel repeated
  rep = Cout ft fs^2 / Cin times, the Cout ft fs^2 channels read as (c, a, b, d) -- c major,
  d minor -- and unfolded to time ft t + a, rows fs h + b, columns fs w + d; on the first
  pass the first ft - 1 output frames are dropped (matching the time conv's 2T - 1 frames).

Layouts: activations (N, T, H, W, C).
"""
from __future__ import annotations

import numpy as np


def time_upsample(x, weight, cache=None, bias=None, first=False):
    """Temporal x2: returns (out (N, first + 2 nf, H, W, C) float64, cache_out (N, 2, H, W, C)).

    nf = T - first frames of x go through the causal time conv:
      P = cat(cache, x[:, first:]) along time (cache zeros if None),
      y[n, i, h, w, k] = bias[k] + sum_{dt in 0..2} sum_c weight[k, dt, c] * P[n, i + dt, h, w, c];
    out[:, first + 2 i + s] = y[:, i, ..., s C : (s + 1) C]; with first, out[:, 0] = x[:, 0].
    cache_out = P[:, nf : nf + 2] (the cache itself when nf = 0).
    """
    x = np.asarray(x, dtype=np.float64)
    n, t, h, w, c = x.shape
    start = 1 if first else 0
    nf = t - start
    wt = np.asarray(weight, dtype=np.float64)
    assert wt.shape == (2 * c, 3, c)
    if cache is None:
        cache = np.zeros((n, 2, h, w, c))
    cache = np.asarray(cache, dtype=np.float64)
    p = np.concatenate([cache, x[:, start:]], axis=1)            # (N, nf + 2, H, W, C)
    y = np.zeros((n, nf, h, w, 2 * c))
    for dt in range(3):
        y += (p[:, dt:dt + nf].reshape(-1, c) @ wt[:, dt, :].T).reshape(n, nf, h, w, 2 * c)
    if bias is not None:
        y += np.asarray(bias, np.float32).astype(np.float64)
    out = np.zeros((n, start + 2 * nf, h, w, c))
    if first:
        out[:, 0] = x[:, 0]
    out[:, start::2] = y[..., :c]
    out[:, start + 1::2] = y[..., c:]
    return out, p[:, nf:nf + 2].copy()


def time_upsample_at(x, weight, cache, bias, first, positions):
    """Outputs of time_upsample at sampled (n, f, h, w) of the output, (S, C) float64."""
    x = np.asarray(x)
    _, _, _, _, c = x.shape
    start = 1 if first else 0
    pos = np.asarray(positions, dtype=np.int64)
    wt = np.asarray(weight, dtype=np.float64)
    out = np.zeros((pos.shape[0], c))
    for r, (n, f, h, w) in enumerate(pos):
        if first and f == 0:
            out[r] = x[n, 0, h, w]
            continue
        i, s = divmod(int(f) - start, 2)
        acc = np.zeros(c) if bias is None else np.asarray(bias, np.float32).astype(np.float64)[s * c:(s + 1) * c]
        for dt in range(3):
            j = i + dt - 2                                        # frame of x[:, start:], < 0: cache
            if j >= 0:
                v = np.asarray(x[n, start + j, h, w], dtype=np.float64)
            elif cache is not None:
                v = np.asarray(cache[n, j + 2, h, w], dtype=np.float64)
            else:
                continue
            acc = acc + wt[s * c:(s + 1) * c, dt, :] @ v
        out[r] = acc
    return out


def dup_up3d(x, cout: int, ft: int, fs: int, first=False):
    """DupUp3D: (N, T, H, W, Cin) -> (N, ft T - first (ft - 1), fs H, fs W, Cout) float64.

    out[n, ft t + a, fs h + b, fs w + d, c] = x[n, t, h, w, (((c ft + a) fs + b) fs + d) // rep],
    rep = Cout ft fs^2 / Cin: built as the channel repeat followed by the unfold.
    """
    x = np.asarray(x, dtype=np.float64)
    n, t, h, w, cin = x.shape
    f = ft * fs * fs
    assert (cout * f) % cin == 0
    rep = cout * f // cin
    v = np.repeat(x, rep, axis=-1)                                # channel j from j // rep
    v = v.reshape(n, t, h, w, cout, ft, fs, fs)                   # j = ((c ft + a) fs + b) fs + d
    v = v.transpose(0, 1, 5, 2, 6, 3, 7, 4)                       # n, t, a, h, b, w, d, c
    v = v.reshape(n, t * ft, h * fs, w * fs, cout)
    return v[:, ft - 1:] if first else v


def dup_up3d_at(x, cout: int, ft: int, fs: int, first, positions):
    """dup_up3d at sampled output positions (n, f, Y, X), (S, Cout): the index formula."""
    x = np.asarray(x)
    cin = x.shape[-1]
    rep = cout * ft * fs * fs // cin
    pos = np.asarray(positions, dtype=np.int64)
    f = pos[:, 1] + (ft - 1 if first else 0)
    t, a = f // ft, f % ft
    h, b = pos[:, 2] // fs, pos[:, 2] % fs
    w, d = pos[:, 3] // fs, pos[:, 3] % fs
    c = np.arange(cout)
    j = ((c[None, :] * ft + a[:, None]) * fs + b[:, None]) * fs + d[:, None]
    rows = np.asarray(x[pos[:, 0], t, h, w], dtype=np.float64)    # (S, Cin)
    return np.take_along_axis(rows, j // rep, axis=1)

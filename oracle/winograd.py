"""Winograd F(4x4, 3x3) form of the causal 3x3x3 convolution, in float64 (test infrastructure only).

Page: FastVideo ``wan22_vae_decode/solution/binding.cpp`` --
* prepare(): the F(4x4,3x3) weight transform of the up blocks' spatial 3x3 taps with a 6x3
  matrix G; each of the 6 x 6 = 36 transformed components keeps the causal 3-tap temporal
  convolution (the sums are formed in fp32 and stored in bf16 there);
* Decoder::conv: only the expensive spatial 3x3 convolutions go through Winograd -- the
  padded input is transformed, one 3-tap temporal convolution runs per component, and an
  epilogue forms the output (with bias and residual).

The pages print G only. Its rows are the Lagrange weights of the interpolation points
0, 1, -1, 2, -2 and the point at infinity (row a of G evaluates a 3-tap filter polynomial
at point a, scaled). The input and output transforms of the same construction are the
ones of Lavin and Gray ("Fast Algorithms for Convolutional Neural Networks", CVPR 2016):
A^T (4 x 6) evaluates the 4 output taps at the points (powers 0..3, with the infinity
column picking the leading coefficient) and B^T (6 x 6) is the matching input transform.
All three are plain tables here; they are pinned by the identity that the Winograd form
equals the direct convolution (tests/test_oracle_winograd.py).

For one 4 x 4 output tile with top-left output pixel (4i, 4j), the 6 x 6 input patch d
covers rows 4i - 1 .. 4i + 4 and columns 4j - 1 .. 4j + 4 (zero outside the frame), and
per frame tap dt and channel pair (k, c):
    V = B^T d B,   U = G g G^T,   Y = A^T (sum over dt, c of U (.) V) A,
with g the 3 x 3 spatial filter and (.) the elementwise product over the 36 components;
output pixels of a tile that fall outside the frame (H or W not multiples of 4) are
dropped.
"""
from __future__ import annotations

import numpy as np

from . import conv as _conv

# G of the page's prepare() (6 x 3).
G = np.array([[1 / 4, 0, 0],
              [-1 / 6, -1 / 6, -1 / 6],
              [-1 / 6, 1 / 6, -1 / 6],
              [1 / 24, 1 / 12, 1 / 6],
              [1 / 24, -1 / 12, 1 / 6],
              [0, 0, 1]], dtype=np.float64)

# Output transform A^T (4 x 6): output tap m at points 0, 1, -1, 2, -2, and infinity.
AT = np.array([[1, 1, 1, 1, 1, 0],
               [0, 1, -1, 2, -2, 0],
               [0, 1, 1, 4, 4, 0],
               [0, 1, -1, 8, -8, 1]], dtype=np.float64)

# Input transform B^T (6 x 6) of the same points.
BT = np.array([[4, 0, -5, 0, 1, 0],
               [0, -4, -4, 1, 1, 0],
               [0, 4, -4, -1, 1, 0],
               [0, -2, -1, 2, 1, 0],
               [0, 2, -1, -2, 1, 0],
               [0, 4, 0, -5, 0, 1]], dtype=np.float64)


def weight_transform(weight):
    """U[a, b, k, dt, c] = sum_{r, s} G[a, r] G[b, s] w[k, dt, r, s, c], float64.

    ``weight`` is (K, 3, 3, 3, C) with taps (dt, dh, dw); returns (6, 6, K, 3, C)."""
    w = np.asarray(weight, dtype=np.float64)
    return np.einsum("ar,bs,ktrsc->abktc", G, G, w)


def tiles(h, w):
    """Tile rows and columns of an H x W frame: ceil(H / 4) x ceil(W / 4)."""
    return (h + 3) // 4, (w + 3) // 4


def input_transform(p):
    """V[a, b, n, f, i, j, c] = (B^T d B)[a, b] of the 6 x 6 patch of tile (i, j) in frame f.

    ``p`` is (N, F, H, W, C) (frames of the causal input P = cat(cache, a)); the patch of tile
    (i, j) covers rows 4i - 1 .. 4i + 4 and columns 4j - 1 .. 4j + 4, zero outside the frame."""
    p = np.asarray(p, dtype=np.float64)
    n, f, h, w, c = p.shape
    th, tw = tiles(h, w)
    pp = np.zeros((n, f, 4 * th + 2, 4 * tw + 2, c))
    pp[:, :, 1:h + 1, 1:w + 1] = p
    # d[n, f, i, j, r, s, c] = pp[n, f, 4i + r, 4j + s, c]
    d = np.empty((n, f, th, tw, 6, 6, c))
    for r in range(6):
        for s in range(6):
            d[:, :, :, :, r, s] = pp[:, :, r:r + 4 * th:4, s:s + 4 * tw:4]
    return np.einsum("ar,bs,nfijrsc->abnfijc", BT, BT, d)


def output_transform(m):
    """Y[n, t, 4i + y, 4j + x, k] = (A^T M A)[y, x] of the 36 components M[a, b, n, t, i, j, k]."""
    y = np.einsum("ya,xb,abntijk->ntiyjxk", AT, AT, np.asarray(m, dtype=np.float64))
    n, t, th, _, tw, _, k = y.shape
    return y.reshape(n, t, 4 * th, 4 * tw, k)


def causal_conv3d(a, weight, cache=None, bias=None, residual=None):
    """The causal 3x3x3 convolution through F(4x4,3x3), float64.

    M[a, b, n, t, i, j, k] = sum_{dt, c} U[a, b, k, dt, c] V[a, b, n, t + dt, i, j, c] over the
    frames of P = cat(cache, a); Y = A^T M A per tile, cropped to H x W, + bias + residual.
    Returns (out (N, T, H, W, K), cache_out = P[:, T:T+2]) as oracle.conv.causal_conv3d."""
    p = _conv.causal_input(a, cache)
    n, t2, h, w, c = p.shape
    t = t2 - 2
    u = weight_transform(weight)
    v = input_transform(p)
    m = np.zeros((6, 6, n, t) + v.shape[4:6] + (u.shape[2],))
    for dt in range(3):
        m += np.einsum("abkc,abntijc->abntijk", u[:, :, :, dt], v[:, :, :, dt:dt + t])
    out = output_transform(m)[:, :, :h, :w]
    if bias is not None:
        out = out + np.asarray(bias, np.float32).astype(np.float64)
    if residual is not None:
        out = out + np.asarray(residual, dtype=np.float64)
    return out, p[:, t:t + 2].copy()

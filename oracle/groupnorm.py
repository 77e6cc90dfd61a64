"""GroupNorm + SiLU, the plain definition in float64 (test infrastructure only).

Follows the WanGP page ``shared/kernels/group_norm_silu.py``: its docstring
(GroupNorm and SiLU computed in higher precision, rounded once to the 16-bit
output) and its apply kernel (the variance is the mean of squared deviations,
i.e. divided by the group length; rstd = 1 / sqrt(var + eps); y = x_hat *
weight + bias; out = y * sigmoid(y)).

Layout: channels-last (N, T, H, W, C); group g holds channels
[g * C/G, (g + 1) * C/G) and all positions of one sample. Statistics cover the
frames passed in only (one pass of the decoder), not the causal cache.
"""
from __future__ import annotations

import numpy as np

_CHUNK_POSITIONS = 1 << 20


def _as_f64_chunks(x, start, stop):
    """Positions [start, stop) of a (N, P, C) view, as float64."""
    return np.asarray(x[:, start:stop, :], dtype=np.float64)


def group_stats(x, groups: int):
    """Mean and biased variance per (sample, group), both float64 arrays (N, G).

    ``x`` holds exact bf16 values (any float dtype) with channels last. Two
    passes: the mean is a compensated (Neumaier) sum of per-chunk float64 sums
    divided by the group length L; the variance is sum((x - mean)**2) / L.
    """
    x = np.asarray(x)
    n = x.shape[0]
    c = x.shape[-1]
    assert c % groups == 0
    cg = c // groups
    xv = x.reshape(n, -1, c)
    npos = xv.shape[1]
    length = npos * cg

    total = np.zeros((n, groups))
    comp = np.zeros((n, groups))
    for s in range(0, npos, _CHUNK_POSITIONS):
        part = _as_f64_chunks(xv, s, min(npos, s + _CHUNK_POSITIONS))
        ps = part.reshape(n, -1, groups, cg).sum(axis=(1, 3))
        t = total + ps                       # Neumaier: keep the lost low part in comp
        comp += np.where(np.abs(total) >= np.abs(ps), (total - t) + ps, (ps - t) + total)
        total = t
    mean = (total + comp) / length

    sq = np.zeros((n, groups))
    for s in range(0, npos, _CHUNK_POSITIONS):
        part = _as_f64_chunks(xv, s, min(npos, s + _CHUNK_POSITIONS)).reshape(n, -1, groups, cg)
        d = part - mean[:, None, :, None]
        sq += (d * d).sum(axis=(1, 3))
    var = sq / length
    return mean, var


def silu(z):
    """z * sigmoid(z) = z / (1 + e^-z) in float64 (e^-z may overflow to inf: the result is then -0)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def normalize(x, mean, var, gamma, beta, eps: float, groups: int):
    """Pre-activation z = (x - mean_g) / sqrt(var_g + eps) * gamma_c + beta_c, float64.

    ``x`` has channels last and a leading sample axis matching ``mean``/``var``
    (N, G); any axes in between are positions (or gathered neighbourhoods).
    ``gamma``/``beta`` are the fp32 affine parameters, ``eps`` is taken as the
    float32 value the library receives and widened exactly.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    c = x.shape[-1]
    cg = c // groups
    eps64 = float(np.float32(eps))
    m = np.repeat(np.asarray(mean, np.float64), cg, axis=1)      # (N, C)
    v = np.repeat(np.asarray(var, np.float64), cg, axis=1)
    shape = (n,) + (1,) * (x.ndim - 2) + (c,)
    xhat = (x - m.reshape(shape)) / np.sqrt(v.reshape(shape) + eps64)
    g = np.asarray(gamma, np.float32).astype(np.float64)
    b = np.asarray(beta, np.float32).astype(np.float64)
    return xhat * g + b


def gn_silu(x, groups: int, gamma, beta, eps: float, stats=None):
    """silu(group_norm(x)) in float64, unrounded. Returns (out, (mean, var))."""
    if stats is None:
        stats = group_stats(x, groups)
    mean, var = stats
    return silu(normalize(x, mean, var, gamma, beta, eps, groups)), stats

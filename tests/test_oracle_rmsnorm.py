"""Pins of the oracle's RMS norm + SiLU (CPU only).

Against: closed forms (a constant position, the zero vector), exact scale invariance,
a pure-Python evaluation on a tiny input, per-position independence, and PyTorch's own
float64 ``rms_norm`` and ``silu`` as an independent library routine.
"""
import math

import numpy as np
import pytest
import torch

import synthgen as sg
from oracle import groupnorm, rmsnorm


def _x(shape, seed=0, mean=0.0):
    return sg.normal(shape, seed, sg.X, mean=mean).float().numpy().astype(np.float64)


def _g(c, seed=0):
    return sg.normal((c,), seed, sg.GAMMA1, std=0.1, mean=1.0, dtype=torch.float32).numpy().astype(np.float64)


def test_constant_position_closed_form():
    # x = c at every channel, eps = 0: rms = |c|, so z = sign(c) * gain exactly
    g = _g(64)
    for c in (1.5, -0.3125, 96.0, -2.0 ** -20):
        x = np.full((1, 1, 1, 2, 64), c)
        out = rmsnorm.rms_silu(x, g, 0.0)
        want = groupnorm.silu(np.sign(c) * g)
        assert np.array_equal(out, np.broadcast_to(want, out.shape))


def test_zero_vector():
    out = rmsnorm.rms_silu(np.zeros((1, 2, 1, 1, 32)), _g(32), 1e-5)
    assert np.array_equal(out, np.zeros_like(out))


def test_scale_invariance():
    x, g = _x((1, 2, 3, 5, 128), 1), _g(128, 1)
    base = rmsnorm.rms_silu(x, g, 0.0)
    for k in (-7, 3, 20):           # powers of two: every step is exact
        assert np.array_equal(rmsnorm.rms_silu(x * 2.0 ** k, g, 0.0), base)
    np.testing.assert_allclose(rmsnorm.rms_silu(x * 3.0, g, 0.0), base, rtol=4e-15, atol=1e-300)


def test_positions_independent():
    x, g = _x((1, 2, 3, 4, 64), 2), _g(64, 2)
    base = rmsnorm.rms_silu(x, g, 1e-6)
    x2 = x.copy()
    x2[0, 1, 2, 3] *= -4.0
    out = rmsnorm.rms_silu(x2, g, 1e-6)
    changed = np.any(out != base, axis=-1)
    assert changed[0, 1, 2, 3] and changed.sum() == 1


def test_pure_python_tiny():
    x, g, eps = _x((1, 2, 2, 3, 8), 3, 0.5), _g(8, 3), 1e-3
    out = rmsnorm.rms_silu(x, g, eps)
    for idx in np.ndindex(*x.shape[:-1]):
        v = [float(t) for t in x[idx]]
        ms = math.fsum(t * t for t in v) / len(v)
        r = math.sqrt(ms + eps)
        for c in range(len(v)):
            z = v[c] * float(g[c]) / r
            want = z / (1.0 + math.exp(-z))
            assert abs(out[idx][c] - want) <= 2e-16 * max(1.0, abs(want))


@pytest.mark.parametrize("shape,eps", [((1, 3, 4, 4, 64), 1e-5), ((2, 2, 5, 3, 256), 1e-6),
                                       ((1, 1, 2, 7, 1024), 1e-5)])
def test_against_torch_rms_norm_fp64(shape, eps):
    x, g = _x(shape, shape[-1], mean=0.3), _g(shape[-1], shape[-1])
    xt, gt = torch.from_numpy(x), torch.from_numpy(g)
    want = torch.nn.functional.silu(torch.nn.functional.rms_norm(xt, (shape[-1],), weight=gt, eps=eps)).numpy()
    np.testing.assert_allclose(rmsnorm.rms_silu(x, g, eps), want, rtol=1e-14, atol=1e-14)


def test_rstd_closed_forms_and_exact_tiny():
    """rms_rstd: a constant position of a power of two with eps = 0 gives 1/|c| exactly; a tiny
    input against its exact rational mean of squares (Fractions), within one rounding of the
    square root and one of the division."""
    from fractions import Fraction
    for c in (0.5, -4.0, 2.0 ** -10):
        r = rmsnorm.rms_rstd(np.full((2, 64), c), 0.0)
        assert np.array_equal(r, np.full(2, 1.0 / abs(c)))
    x = _x((1, 1, 2, 3, 8), 7)
    eps = 1e-5
    r = rmsnorm.rms_rstd(x, eps)
    assert r.shape == (1, 1, 2, 3)
    for idx in np.ndindex(r.shape):
        ms = sum(Fraction(v) ** 2 for v in x[idx]) / 8 + Fraction(eps)
        want = 1.0 / math.sqrt(float(ms))
        assert abs(r[idx] - want) <= 4e-16 * want


def test_rstd_against_torch_rsqrt_fp64():
    """Against torch's float64 rsqrt of the mean of squares (an independent library routine), and
    rms_silu as the SiLU of x * gain * rstd (the two forms of the same norm, to fp64 rounding)."""
    x, g = _x((2, 2, 5, 3, 256), 3, mean=0.3), _g(256, 3)
    r = rmsnorm.rms_rstd(x, 1e-6)
    t = torch.rsqrt(torch.from_numpy(x).pow(2).mean(dim=-1) + 1e-6).numpy()
    assert np.allclose(r, t, rtol=1e-14, atol=0)
    via = groupnorm.silu(x * g * r[..., None])
    assert np.allclose(via, rmsnorm.rms_silu(x, g, 1e-6), rtol=1e-13, atol=1e-300)

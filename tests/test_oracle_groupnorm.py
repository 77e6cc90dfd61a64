"""Pins of the oracle's GroupNorm + SiLU (CPU only).

Against: exact rational arithmetic on tiny inputs, the normalisation
invariants, closed-form special cases, and PyTorch's own float64
``group_norm`` / ``silu`` as an independent library routine.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synthgen as sg
from oracle import bf16, groupnorm


def _tiny(seed=0, shape=(1, 3, 4, 4, 64), offset=0.0):
    x = sg.normal(shape, seed, sg.X, mean=offset)
    return x.float().numpy().astype(np.float64)


def test_stats_exact_rational_tiny():
    x = _tiny()
    g = 32
    mean, var = groupnorm.group_stats(x, g)
    xv = x.reshape(1, -1, g, 2)
    for gi in range(g):
        vals = [Fraction(float(v)) for v in xv[0, :, gi, :].ravel()]
        m = sum(vals) / len(vals)
        v = sum((u - m) ** 2 for u in vals) / len(vals)
        assert mean[0, gi] == float(m)                      # exact sum of bf16 values, one rounding
        assert abs(var[0, gi] - float(v)) <= 1e-15 * float(v)


def test_stats_multi_chunk_exact_rational(monkeypatch):
    """More positions than one chunk (8 chunks of 5 positions, the last ragged, two samples):
    the per-chunk sums are combined by the compensated step, the variance pass runs chunk by
    chunk; against exact rational arithmetic."""
    monkeypatch.setattr(groupnorm, "_CHUNK_POSITIONS", 5)
    x = _tiny(seed=5, shape=(2, 3, 4, 3, 16), offset=300.0)        # 36 positions per sample
    g = 4
    mean, var = groupnorm.group_stats(x, g)
    xv = x.reshape(2, -1, g, 4)
    for n in range(2):
        for gi in range(g):
            vals = [Fraction(float(v)) for v in xv[n, :, gi, :].ravel()]
            m = sum(vals) / len(vals)
            v = sum((u - m) ** 2 for u in vals) / len(vals)
            assert abs(mean[n, gi] - float(m)) <= 1e-15 * abs(float(m))
            assert abs(var[n, gi] - float(v)) <= 1e-13 * float(v)


def test_stats_chunk_sums_compensated(monkeypatch):
    """One position per chunk, so that every chunk sum is one exact value: the group's values
    2^60, 1, -2^60, 1 have mean 1/2 exactly. A plain running fp64 sum loses the first 1 against
    2^60 and gives 1/4; the compensated combination must keep it."""
    monkeypatch.setattr(groupnorm, "_CHUNK_POSITIONS", 1)
    x = np.array([2.0 ** 60, 1.0, -2.0 ** 60, 1.0]).reshape(1, 4, 1, 1, 1) * np.ones((1, 1, 1, 1, 8))
    mean, var = groupnorm.group_stats(x, 8)
    assert np.all(mean == 0.5)
    half = Fraction(1, 2)
    exact = ((2 ** 60 - half) ** 2 + (-(2 ** 60) - half) ** 2 + 2 * half ** 2) / 4
    assert np.allclose(var, float(exact), rtol=1e-15, atol=0)


def test_stats_large_mean_no_cancellation():
    # A group offset by 1000 with unit spread: the two-pass variance is still ~1.
    x = _tiny(offset=1000.0)
    mean, var = groupnorm.group_stats(x, 32)
    xv = x.reshape(1, -1, 32, 2)
    for gi in (0, 7, 31):
        vals = [Fraction(float(v)) for v in xv[0, :, gi, :].ravel()]
        m = sum(vals) / len(vals)
        v = sum((u - m) ** 2 for u in vals) / len(vals)
        assert abs(var[0, gi] - float(v)) <= 1e-12 * float(v)


def test_normalized_invariants():
    x = _tiny(seed=3, shape=(2, 2, 5, 3, 32))
    g = 8
    mean, var = groupnorm.group_stats(x, g)
    ones, zeros = np.ones(32, np.float32), np.zeros(32, np.float32)
    eps = 1e-5
    z = groupnorm.normalize(x, mean, var, ones, zeros, eps, g)     # affine = identity
    zv = z.reshape(2, -1, g, 4)
    assert np.abs(zv.mean(axis=(1, 3))).max() <= 1e-12
    m2 = (zv ** 2).mean(axis=(1, 3))
    eps64 = float(np.float32(eps))
    assert np.allclose(m2, var / (var + eps64), rtol=1e-12, atol=0)


def test_constant_group_and_zero_gamma_give_silu_beta():
    x = np.full((1, 2, 3, 3, 16), 0.75)
    beta = np.linspace(-2, 2, 16).astype(np.float32)
    gamma = np.ones(16, np.float32)
    out, (mean, var) = groupnorm.gn_silu(x, 4, gamma, beta, 1e-5)
    assert np.all(var == 0) and np.all(mean == 0.75)
    b = beta.astype(np.float64)
    want = b / (1 + np.exp(-b))
    assert np.allclose(out, np.broadcast_to(want, out.shape), rtol=0, atol=0)
    y = _tiny(shape=(1, 2, 3, 3, 16))
    out2, _ = groupnorm.gn_silu(y, 4, np.zeros(16, np.float32), beta, 1e-5)
    assert np.array_equal(out2, np.broadcast_to(want, out2.shape))


def test_silu_closed_forms():
    z = np.array([0.0, 1e-300, 50.0, -50.0, 800.0, -800.0, 2.5])
    s = groupnorm.silu(z)
    assert s[0] == 0 and s[1] == 5e-301
    assert s[2] == 50.0 and s[4] == 800.0
    assert abs(s[3] - (-50.0 * np.exp(-50.0))) <= 1e-15 * abs(s[3])
    assert s[5] == 0.0
    # silu(z) - silu(-z) = z
    assert abs((s[6] - groupnorm.silu(-2.5)) - 2.5) <= 1e-15


@pytest.mark.parametrize("shape,groups", [((1, 3, 16, 16, 64), 32), ((2, 2, 6, 5, 48), 6)])
def test_against_torch_group_norm_fp64(shape, groups):
    x = sg.normal(shape, 7, sg.X, mean=0.3)
    c = shape[-1]
    gamma = sg.normal((c,), 7, sg.GAMMA1, std=0.1, mean=1.0, dtype=torch.float32)
    beta = sg.normal((c,), 7, sg.BETA1, std=0.1, dtype=torch.float32)
    eps = 1e-5
    out, _ = groupnorm.gn_silu(x.float().numpy(), groups, gamma.numpy(), beta.numpy(), eps)
    xt = x.double().permute(0, 4, 1, 2, 3)                      # NCTHW for torch
    ref = torch.nn.functional.group_norm(xt, groups, gamma.double(), beta.double(),
                                         float(np.float32(eps)))
    ref = torch.nn.functional.silu(ref).permute(0, 2, 3, 4, 1).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_rounding_of_output_is_single():
    x = _tiny()
    gamma = np.ones(64, np.float32)
    beta = np.zeros(64, np.float32)
    out, _ = groupnorm.gn_silu(x, 32, gamma, beta, 1e-5)
    bits = bf16.round_rne(out)
    back = bf16.decode(bits)
    # every result is within half a bf16 quantum of the float64 value
    _, e = np.frexp(np.abs(out))
    q = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    assert np.all(np.abs(back - out) <= q / 2)

"""GroupNorm + SiLU on the GPU vs the fp64 oracle (gn_silu_stats, gn_silu_apply).

Gate: every output within 1 bf16 ulp of the oracle's fp64 result rounded once;
statistics within 1e-12 (relative) of the oracle's two-pass fp64 values.
"""
import numpy as np
import pytest
import torch

import silu_gn_amd as sga
import synthgen as sg
from oracle import groupnorm as ogn
from synthgen.workloads import WORKLOADS
from tests.helpers import bits, ulp_report, vals32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _params(c, seed):
    gamma = sg.normal((c,), seed, sg.GAMMA1, std=0.1, mean=1.0, dtype=torch.float32)
    beta = sg.normal((c,), seed, sg.BETA1, std=0.1, dtype=torch.float32)
    return gamma, beta


def _run_and_check(x_cpu, groups, gamma, beta, eps=1e-5, sample=None, what=""):
    print("case", what, tuple(x_cpu.shape), "G=%d" % groups, flush=True)
    x = x_cpu.to(DEV)
    stats = sga.gn_silu_stats(x, groups)
    y = sga.gn_silu_apply(x, groups, stats, gamma.to(DEV), beta.to(DEV), eps)
    torch.cuda.synchronize()
    xv = vals32(x_cpu)
    mean, var = ogn.group_stats(xv, groups)
    st = stats.cpu().numpy()
    assert np.allclose(st[..., 0], mean, rtol=1e-12, atol=1e-13), np.abs(st[..., 0] - mean).max()
    assert np.allclose(st[..., 1], var, rtol=1e-12, atol=1e-15), np.abs(st[..., 1] / var - 1).max()
    if sample is not None:
        xv = xv.reshape(xv.shape[0], -1, xv.shape[-1])[:, sample].astype(np.float64)
        yb = bits(y.reshape(y.shape[0], -1, y.shape[-1])[:, torch.from_numpy(sample).to(y.device)])
    else:
        yb = bits(y)
    o, _ = ogn.gn_silu(xv, groups, gamma.numpy(), beta.numpy(), eps, stats=(mean, var))
    mx, exact = ulp_report(yb, o)
    print("  max ulp %d, exact %.5f" % (mx, exact), flush=True)
    assert mx <= 1
    return stats, y


@pytest.mark.parametrize("shape,groups", [
    ((1, 3, 16, 16, 64), 32),      # C/G = 2
    ((2, 3, 5, 7, 64), 16),        # C/G = 4, two samples, ragged positions
    ((1, 1, 1, 3, 64), 64),        # C/G = 1, 3 positions
    ((1, 2, 9, 11, 256), 32),      # C/G = 8
    ((1, 4, 6, 13, 1024), 32),     # C/G = 32
    ((3, 2, 3, 5, 512), 4),        # C/G = 128
    ((1, 5, 17, 19, 2048), 32),    # largest C
])
def test_gn_small_shapes(shape, groups):
    x = sg.normal(shape, 11, sg.X, mean=0.25)
    gamma, beta = _params(shape[-1], 11)
    _run_and_check(x, groups, gamma, beta, what="small")


def test_gn_large_offsets_and_spread():
    # per-channel offsets of +-1000 and a few huge / tiny magnitudes
    c = 256
    off = sg.uniform((c,), 5, sg.OFFSETS, -1000.0, 1000.0)
    x = sg.normal((1, 2, 16, 24, c), 5, sg.X, std=3.0, mean=off)
    gamma, beta = _params(c, 5)
    _run_and_check(x, 32, gamma, beta, what="offsets")


def test_gn_extreme_preactivations():
    # gamma large enough that z reaches -100 .. +100: the overflow-free SiLU path and
    # bf16 subnormal outputs (z e^z near 1e-40) are exercised.
    c = 64
    x = sg.normal((1, 2, 8, 8, c), 6, sg.X)
    gamma = torch.linspace(1.0, 40.0, c, dtype=torch.float32)
    beta = torch.linspace(-60.0, 10.0, c, dtype=torch.float32)
    _run_and_check(x, 8, gamma, beta, what="extreme")


def test_gn_constant_groups():
    x = torch.full((1, 2, 4, 4, 64), 1.5, dtype=torch.bfloat16)
    gamma, beta = _params(64, 3)
    stats, y = _run_and_check(x, 32, gamma, beta, what="constant")
    assert torch.all(stats[..., 1] == 0)


def test_gn_in_place_and_deterministic():
    x = sg.normal((1, 3, 20, 30, 256), 9, sg.X).to(DEV)
    gamma, beta = (t.to(DEV) for t in _params(256, 9))
    s1 = sga.gn_silu_stats(x, 32)
    s2 = sga.gn_silu_stats(x, 32)
    assert torch.equal(s1, s2)
    y1 = sga.gn_silu_apply(x, 32, s1, gamma, beta, 1e-5)
    x2 = x.clone()
    sga.gn_silu_apply(x2, 32, s1, gamma, beta, 1e-5, y=x2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), x2.view(torch.int16))


@pytest.mark.parametrize("idx", [1, 2])
def test_gn_workload_full(idx):
    wl = WORKLOADS[idx]
    x = wl.x()
    _run_and_check(x, wl.groups, wl.gamma(), wl.beta(), wl.eps, what=wl.name)


@pytest.mark.slow
@pytest.mark.parametrize("idx", [3, 4, 5])
def test_gn_workload_large_sampled(idx):
    """Full-size tensors: statistics checked exactly, the output on 2^18 sampled positions."""
    wl = WORKLOADS[idx]
    if idx == 3:
        shape = (1, wl.t, 2 * wl.h, 2 * wl.w, wl.c)    # the upsampled tensor the block normalises
        x = sg.normal(shape, wl.seed, sg.X_PREV, device=DEV).cpu()
    else:
        x = wl.x(device=DEV).cpu()
    npos = x.numel() // x.shape[-1]
    sample = np.sort(np.random.default_rng(idx).choice(npos, 1 << 18, replace=False))
    _run_and_check(x, wl.groups, wl.gamma(), wl.beta(), wl.eps, sample=sample, what=wl.name)

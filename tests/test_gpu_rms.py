"""RMS norm + SiLU on the GPU vs the fp64 oracle (rms_silu).

Gate: every output within 1 bf16 ulp of the oracle's fp64 result rounded once.
"""
import numpy as np
import pytest
import torch

import silu_gn_amd as sga
import synthgen as sg
from oracle import rmsnorm as orms
from synthgen.workloads import WORKLOADS
from tests.helpers import bits, ulp_report, vals32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gain(c, seed):
    return sg.normal((c,), seed, sg.GAMMA1, std=0.1, mean=1.0, dtype=torch.float32)


def _check(x_cpu, gain, eps=1e-6, sample=None, what=""):
    print("case", what, tuple(x_cpu.shape), flush=True)
    x = x_cpu.to(DEV)
    y = sga.rms_silu(x, gain.to(DEV), eps)
    torch.cuda.synchronize()
    c = x_cpu.shape[-1]
    xv = vals32(x_cpu).reshape(-1, c)
    yb = bits(y).reshape(-1, c)
    if sample is not None:
        xv, yb = xv[sample], yb[sample]
    o = orms.rms_silu(xv.astype(np.float64), gain.numpy(), eps)
    mx, exact = ulp_report(yb, o)
    print("  max ulp %d, exact %.5f" % (mx, exact), flush=True)
    assert mx <= 1
    return y


# Every kernel variant (C/8 packets: 8, 16, 32, 64 lanes per position, then 2, 4, 8 packets
# per lane), ragged position counts that leave a block partly empty.
@pytest.mark.parametrize("shape", [
    (1, 1, 1, 3, 64),
    (2, 3, 5, 7, 64),
    (1, 2, 9, 11, 128),
    (1, 3, 7, 5, 192),
    (2, 2, 6, 13, 256),
    (1, 2, 5, 3, 320),
    (1, 4, 6, 13, 512),
    (1, 2, 7, 9, 1024),
    (1, 1, 17, 19, 2048),
    (1, 1, 3, 5, 4096),
])
def test_rms_small_shapes(shape):
    x = sg.normal(shape, 21, sg.X, mean=0.25)
    _check(x, _gain(shape[-1], 21), what="small")


def test_rms_extremes():
    # large and tiny per-channel scales, a zero position (0 * gain / sqrt(eps) = 0) and
    # gains big enough to reach the SiLU tails
    c = 256
    x = sg.normal((1, 2, 8, 8, c), 22, sg.X, std=1.0)
    x = x * torch.logspace(-3, 3, c).to(torch.bfloat16)
    x[0, 0, 0, 0] = 0
    gain = torch.linspace(-30.0, 30.0, c, dtype=torch.float32)
    _check(x, gain, eps=1e-5, what="extremes")


def test_rms_in_place_and_deterministic():
    x = sg.normal((1, 3, 20, 30, 256), 23, sg.X).to(DEV)
    gain = _gain(256, 23).to(DEV)
    y1 = sga.rms_silu(x, gain, 1e-6)
    y2 = sga.rms_silu(x, gain, 1e-6)
    x2 = x.clone()
    sga.rms_silu(x2, gain, 1e-6, y=x2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), x2.view(torch.int16))


@pytest.mark.slow
def test_rms_output_head_full_sampled():
    """The output head's input at full size (C=256, 16x352x624); 2^18 sampled positions."""
    wl = WORKLOADS[5]
    x = wl.x(device=DEV).cpu()
    npos = x.numel() // x.shape[-1]
    sample = np.sort(np.random.default_rng(5).choice(npos, 1 << 18, replace=False))
    sample[0], sample[-1] = 0, npos - 1
    _check(x, wl.gamma(), eps=1e-6, sample=sample, what=wl.name)


# ---------------------------------------------------------------- the norm in the consumer's operand load
@pytest.mark.parametrize("shape", [(1, 1, 1, 3, 64), (2, 3, 5, 7, 64), (1, 3, 7, 5, 192), (2, 2, 6, 13, 256),
                                   (1, 2, 7, 9, 1024), (1, 1, 3, 5, 4096)])
def test_rms_rstd_vs_oracle(shape):
    """rms_silu_rstd: each position's fp64 factor against the oracle's (exact squares summed in
    another order: equal to a few fp64 ulps)."""
    from oracle import rmsnorm as orms2
    print("case rstd", shape, flush=True)
    x = sg.normal(shape, 31, sg.X, mean=0.25)
    r = sga.rms_silu_rstd(x.to(DEV), 1e-6)
    torch.cuda.synchronize()
    want = orms2.rms_rstd(vals32(x).astype(np.float64), 1e-6)
    assert np.allclose(r.cpu().numpy(), want, rtol=1e-14, atol=0)


def _w(k, c, seed):
    import math
    return sg.normal((k, 3, 3, 3, c), seed, sg.W1, std=1 / math.sqrt(27 * c))


@pytest.mark.parametrize("n,t,h,w,c,k,cache,bias,res", [
    (1, 3, 8, 10, 64, 64, True, True, False),      # K <= 128: the generic tile on both sides
    (2, 2, 5, 13, 128, 256, True, False, True),    # K > 128: the slab kernel unfused, two samples
    (1, 1, 6, 7, 256, 12, False, True, True),      # T = 1 without a cache, K = 12
    (1, 2, 9, 33, 512, 320, True, True, True),     # two N tiles, the second ragged
    (1, 2, 1, 1, 64, 256, True, True, False),      # a single pixel
    (1, 2, 3, 4, 2048, 64, True, False, False),    # the largest C it takes
])
def test_conv_rms_input_equals_rms_then_conv(n, t, h, w, c, k, cache, bias, res):
    """causal_conv3d_rms_input: y and the activated cache_out bitwise those of rms_silu followed by
    causal_conv3d, and y against the oracle (its RMS norm rounded once, then its conv)."""
    from oracle import bf16 as obf16
    from oracle import conv as oconv
    from tests.helpers import assert_conv_close, vals
    print("case conv rms input", (n, t, h, w, c, k, cache, bias, res), flush=True)
    seed = n + t + h + w + c + k + 41
    x = sg.normal((n, t, h, w, c), seed, sg.X, mean=0.2)
    gain = _gain(c, seed)
    wt = _w(k, c, seed)
    ci = sg.normal((n, 2, h, w, c), seed, sg.X_PREV) if cache else None
    b = sg.normal((k,), seed, sg.BETA2, std=0.5, dtype=torch.float32) if bias else None
    r = sg.normal((n, t, h, w, k), seed, sg.GAMMA2) if res else None
    xd, gd, wd = x.to(DEV), gain.to(DEV), wt.to(DEV)
    cd = ci.to(DEV) if cache else None
    bd = b.to(DEV) if bias else None
    rd = r.to(DEV) if res else None
    eps = 1e-6
    a = sga.rms_silu(xd, gd, eps)
    co1 = torch.empty((n, 2, h, w, c), dtype=torch.bfloat16, device=DEV)
    co2 = torch.empty_like(co1)
    y1 = sga.causal_conv3d(a, wd, cd, bd, rd, cache_out=co1)
    rstd = sga.rms_silu_rstd(xd, eps)
    y2 = sga.causal_conv3d_rms_input(xd, wd, rstd, gd, cd, bd, rd, cache_out=co2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(co1.view(torch.int16), co2.view(torch.int16))
    act = obf16.decode(obf16.round_rne(orms.rms_silu(vals(x), gain.numpy(), eps)))
    o, _ = oconv.causal_conv3d(act, vals(wt), vals(ci) if cache else None, b.numpy() if bias else None,
                               vals(r) if res else None)
    assert_conv_close(bits(y2), o, "conv rms input")


@pytest.mark.slow
def test_conv_rms_input_fullres():
    """The full-resolution shape [1,16,352,624,256] -> 256 with a cache and the residual:
    bitwise equal to rms_silu then causal_conv3d (whole tensors, y and cache_out)."""
    wl = WORKLOADS[4]
    print("case conv rms input full-res", flush=True)
    x = wl.x(device=DEV)
    gain, wt = wl.gamma(2, DEV), wl.conv_weight(1, DEV)
    ci = wl.x_prev(DEV)[:, -2:].contiguous()
    a = sga.rms_silu(x, gain, 1e-6)
    co1, co2 = torch.empty_like(ci), torch.empty_like(ci)
    y1 = sga.causal_conv3d(a, wt, ci, residual=x, cache_out=co1)
    del a
    rstd = sga.rms_silu_rstd(x, 1e-6)
    y2 = sga.causal_conv3d_rms_input(x, wt, rstd, gain, ci, residual=x, cache_out=co2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(co1.view(torch.int16), co2.view(torch.int16))

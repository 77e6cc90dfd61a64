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

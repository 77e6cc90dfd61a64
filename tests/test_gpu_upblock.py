"""The rest of an up block on the GPU vs the oracle: the temporal x2 (time_upsample_conv)
and the phase convolutions with the DupUp3D shortcut (upsample2x_conv_phases_shortcut).

Gates: the convolution outputs within the convolution tolerance of the oracle's float64
result; the passed-through first frame and cache_out bit-exact.
"""
import math

import numpy as np
import pytest
import torch

import silu_gn_amd as sga
import synthgen as sg
from oracle import conv as oconv
from oracle import upblock as oup
from synthgen.workloads import WORKLOADS
from tests.helpers import assert_conv_close, bits, sample_positions, vals, vals32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _time_inputs(n, t, h, w, c, cache, bias, seed):
    x = sg.normal((n, t, h, w, c), seed, sg.X)
    wt = sg.normal((2 * c, 3, c), seed, sg.W_TIME, std=1 / math.sqrt(3 * c))
    ci = sg.normal((n, 2, h, w, c), seed, sg.X_PREV) if cache else None
    b = sg.normal((2 * c,), seed, sg.BETA2, std=0.5, dtype=torch.float32) if bias else None
    return x, wt, ci, b


@pytest.mark.parametrize("n,t,h,w,c,first,cache,bias", [
    (1, 3, 5, 7, 64, True, True, True),
    (2, 2, 5, 7, 64, False, False, False),
    (1, 1, 3, 4, 64, True, True, True),        # first pass of one frame: only the copy and the cache
    (2, 1, 3, 4, 64, False, True, True),
    (1, 3, 17, 19, 128, False, True, True),    # two M tiles per frame, the second ragged
    (1, 2, 9, 11, 192, True, True, True),      # K = 384: the second N tile half full
    (2, 3, 4, 5, 256, True, False, False),
    (1, 2, 3, 5, 320, False, True, True),
    (1, 2, 5, 6, 1024, True, True, True),
    (1, 2, 3, 3, 2048, True, True, True),      # the largest C: K = 4096, 16 N tiles
])
def test_time_upsample_small(n, t, h, w, c, first, cache, bias):
    print("case time_upsample", (n, t, h, w, c, first, cache, bias), flush=True)
    x, wt, ci, b = _time_inputs(n, t, h, w, c, cache, bias, seed=t + h + w + c)
    co = torch.empty((n, 2, h, w, c), dtype=torch.bfloat16, device=DEV)
    y = sga.time_upsample_conv(x.to(DEV), wt.to(DEV), first, ci.to(DEV) if cache else None,
                               b.to(DEV) if bias else None, cache_out=co)
    torch.cuda.synchronize()
    o, oc = oup.time_upsample(vals(x), vals(wt), vals(ci) if cache else None, b.numpy() if bias else None, first)
    yb = bits(y)
    assert yb.shape == o.shape
    start = 1 if first else 0
    if first:
        assert np.array_equal(yb[:, 0], bits(x)[:, 0])
    if o.shape[1] > start:
        assert_conv_close(yb[:, start:], o[:, start:], "time_upsample")
    assert np.array_equal(bits(co), bits(torch.from_numpy(oc).to(torch.bfloat16)))


def test_time_upsample_pass_split():
    # two passes carrying the cache give the bits of one pass (fixed accumulation order)
    n, t, h, w, c = 1, 5, 6, 7, 128
    x, wt, _, b = _time_inputs(n, t, h, w, c, False, True, seed=77)
    xd, wd, bd = x.to(DEV), wt.to(DEV), b.to(DEV)
    whole = sga.time_upsample_conv(xd, wd, True, None, bd)
    co = torch.empty((n, 2, h, w, c), dtype=torch.bfloat16, device=DEV)
    a = sga.time_upsample_conv(xd[:, :2].contiguous(), wd, True, None, bd, cache_out=co)
    bb = sga.time_upsample_conv(xd[:, 2:].contiguous(), wd, False, co, bd)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([a, bb], dim=1).view(torch.int16), whole.view(torch.int16))


@pytest.mark.slow
@pytest.mark.parametrize("first", [True, False])
def test_time_upsample_latent_workload_sampled(first):
    """x [1,4,44,78,1024] -> 2048 channels -> y [1,7 or 8,44,78,1024]; sampled positions."""
    wl = WORKLOADS[2]
    n, t, h, w, c = wl.shape
    x = wl.x(device=DEV)
    wt = sg.normal((2 * c, 3, c), wl.seed, sg.W_TIME, std=1 / math.sqrt(3 * c), device=DEV)
    b = sg.normal((2 * c,), wl.seed, sg.BETA2, std=0.5, dtype=torch.float32, device=DEV)
    ci = None if first else wl.x_prev(device=DEV)[:, -2:].contiguous()
    print("case time_upsample latent first=%s" % first, flush=True)
    y = sga.time_upsample_conv(x, wt, first, ci, b)
    torch.cuda.synchronize()
    to = y.shape[1]
    rng = np.random.default_rng(3)
    pos = np.stack([np.zeros(1024, np.int64), rng.integers(0, to, 1024), rng.integers(0, h, 1024),
                    rng.integers(0, w, 1024)], axis=1)
    pos[:4, 1] = [0, 1, to - 2, to - 1]
    o = oup.time_upsample_at(vals32(x), vals(wt.cpu()), vals32(ci) if ci is not None else None, b.cpu().numpy(),
                             first, pos)
    idx = tuple(torch.from_numpy(pos[:, i]) for i in range(4))
    got = bits(y.cpu()[idx])
    if first:
        head = pos[:, 1] == 0
        hp = pos[head]
        xh = x.cpu()[hp[:, 0], 0, hp[:, 2], hp[:, 3]]
        assert np.array_equal(got[head], bits(xh))
        got, o = got[~head], o[~head]
    assert_conv_close(got, o, "time_upsample sampled")


@pytest.mark.parametrize("n,ts,h,w,c,k,cs,ft,first,bias", [
    (1, 2, 3, 5, 64, 64, 64, 2, True, True),
    (1, 2, 3, 5, 64, 64, 128, 2, False, True),      # C_in = 2K: source channels 2c, 2c + 1
    (2, 2, 4, 5, 64, 128, 256, 1, False, False),
    (1, 3, 5, 7, 64, 256, 256, 2, True, True),      # K > 128: the slab kernel's epilogue
    (1, 2, 5, 6, 64, 256, 512, 1, False, True),
    (1, 2, 17, 19, 64, 128, 128, 1, True, True),    # first with ft = 1 drops nothing
    (1, 1, 9, 30, 64, 264, 528, 2, False, True),    # K over two N tiles, the second ragged
    (1, 2, 3, 5, 128, 192, 192, 2, True, False),
])
def test_upsample_shortcut_small(n, ts, h, w, c, k, cs, ft, first, bias):
    t = ft * ts - (ft - 1 if first else 0)
    print("case upsample_shortcut", (n, ts, t, h, w, c, k, cs, ft, first, bias), flush=True)
    seed = ts + h + w + c + k + cs
    x = sg.normal((n, t, h, w, c), seed, sg.X)
    src = sg.normal((n, ts, h, w, cs), seed, sg.X_BLOCK)
    w3 = sg.normal((k, 3, 3, c), seed, sg.W_UP, std=1 / math.sqrt(9 * c))
    b = sg.normal((k,), seed, sg.BETA2, std=0.5, dtype=torch.float32) if bias else None
    wp = sga.upsample2x_prepare_weights(w3).to(DEV)
    y = sga.upsample2x_conv_phases_shortcut(x.to(DEV), wp, src.to(DEV), ft, first, b.to(DEV) if bias else None)
    torch.cuda.synchronize()
    o = oconv.upsample2x_conv(vals(x), vals(w3), b.numpy() if bias else None)
    o = o + oup.dup_up3d(vals(src), k, ft, 2, first)
    assert_conv_close(bits(y), o, "upsample+shortcut")


@pytest.mark.slow
@pytest.mark.parametrize("ft,first", [(1, False), (2, True)])
def test_upsample_shortcut_workload_sampled(ft, first):
    """The upsample block's phases, x [1,T,88,156,512] -> [1,T,176,312,512], plus the shortcut
    of a block input [1,T_in,88,156,512] (T = 8; with ft = 2 and first, T_in = 4 and T = 7)."""
    wl = WORKLOADS[3]
    ts = wl.t if ft == 1 else wl.t // 2
    t = ft * ts - (ft - 1 if first else 0)
    shape = (1, t, wl.h, wl.w, wl.c)
    x = sg.normal(shape, wl.seed, sg.X, device=DEV)
    src = sg.normal((1, ts, wl.h, wl.w, wl.c), wl.seed, sg.X_BLOCK, device=DEV)
    w3 = wl.up_weight()
    wp = sga.upsample2x_prepare_weights(w3).to(DEV)
    print("case upsample_shortcut workload ft=%d first=%s" % (ft, first), flush=True)
    y = sga.upsample2x_conv_phases_shortcut(x, wp, src, ft, first)
    torch.cuda.synchronize()
    pos = sample_positions(t, 2 * wl.h, 2 * wl.w, 16384, seed=6)
    o = oconv.upsample2x_conv_at(vals32(x), vals(w3), pos)
    o = o + oup.dup_up3d_at(vals32(src), wl.c, ft, 2, first, pos)
    idx = tuple(torch.from_numpy(pos[:, i]) for i in range(4))
    assert_conv_close(bits(y.cpu()[idx]), o, "upsample+shortcut sampled")


def test_up_block_chain():
    """An up block's tail on a first pass: the temporal x2 of the resnets' output, then the
    phases with the bias and the DupUp3D shortcut of the block input (ft = 2), against the
    oracle's own composition (its temporal x2 rounded once to bf16 between the steps, where
    the library stores the intermediate)."""
    from oracle import bf16 as obf16
    n, t, h, w, c = 1, 3, 6, 9, 128
    seed = 91
    xin = sg.normal((n, t, h, w, c), seed, sg.X_BLOCK)             # the block's input
    x = sg.normal((n, t, h, w, c), seed, sg.X)                     # the resnets' output
    wt = sg.normal((2 * c, 3, c), seed, sg.W_TIME, std=1 / math.sqrt(3 * c))
    bt = sg.normal((2 * c,), seed, sg.BETA1, std=0.5, dtype=torch.float32)
    w3 = sg.normal((c, 3, 3, c), seed, sg.W_UP, std=1 / math.sqrt(9 * c))
    b3 = sg.normal((c,), seed, sg.BETA2, std=0.5, dtype=torch.float32)
    print("case up block chain", (n, t, h, w, c), flush=True)
    u = sga.time_upsample_conv(x.to(DEV), wt.to(DEV), True, None, bt.to(DEV))
    wp = sga.upsample2x_prepare_weights(w3).to(DEV)
    y = sga.upsample2x_conv_phases_shortcut(u, wp, xin.to(DEV), 2, True, b3.to(DEV))
    torch.cuda.synchronize()
    ou, _ = oup.time_upsample(vals(x), vals(wt), None, bt.numpy(), True)
    assert_conv_close(bits(u)[:, 1:], ou[:, 1:], "chain: temporal x2")
    our = obf16.decode(obf16.round_rne(ou))                        # stored in bf16 between the steps
    o = oconv.upsample2x_conv(our, vals(w3), b3.numpy()) + oup.dup_up3d(vals(xin), c, 2, 2, True)
    assert y.shape == (n, 2 * t - 1, 2 * h, 2 * w, c)
    assert_conv_close(bits(y), o, "chain: phases + shortcut")

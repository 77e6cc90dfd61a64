"""The unfused causal convolution -- the kernel and tiles bench.py times -- against the fp64
oracle, at small shapes in full and at the workloads' full sizes.

Which kernel runs is asked of the library (sgn_conv_plan) and asserted, so each case is
known to cover the tile it is meant to: the slab kernel's 256 x 256 tile (the upsample and
full-resolution blocks) and its 224-row tile (the latent block).

Gate: relative L2 error <= 1e-2 and max abs error <= 4e-2 against the unrounded fp64 oracle
(unit-scale data); cache_out bitwise. At full size the conv parity is stage-wise (each oracle
stage takes the GPU's previous-stage bf16 output as its input) on sampled positions: every
border position of frames {0, 1, T-1} plus seeded interior positions, all K channels each.
GroupNorm+SiLU outputs on the way are checked against the oracle within 1 bf16 ulp.
"""
import math

import numpy as np
import pytest
import torch

import silu_gn_amd as sga
import synthgen as sg
from oracle import bf16 as obf16
from oracle import conv as oconv
from oracle import groupnorm as ogn
from synthgen.workloads import WORKLOADS
from tests.helpers import assert_conv_close, bits, sample_positions, vals, vals32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _w(k, c, seed, tid=sg.W1):
    return sg.normal((k, 3, 3, 3, c), seed, tid, std=1 / math.sqrt(27 * c))


def _plan(shape, k):
    return sga.sgn_conv_plan(sga.SGN_OP_CAUSAL, shape, k)


@pytest.mark.parametrize("shape,k,tile_m", [
    ((1, 16, 64, 64, 64), 256, 256),      # 256 tiles of 256 rows: one full wave of the chip
    ((2, 11, 22, 51, 128), 320, 256),     # ragged M (1122 = 4 x 256 + 98) and N (320 = 256 + 64)
    ((1, 4, 6, 70, 256), 256, 224),       # the 224-row tile, ragged
])
def test_unfused_tile_full(shape, k, tile_m):
    """Every output of the slab kernel's tile against the oracle, with a cache, a bias and a
    residual; cache_out bitwise."""
    plan = _plan(shape, k)
    assert plan["kernel"] == "slab" and plan["tile_m"] == tile_m and plan["tile_n"] == 256, plan
    print("case unfused tile", shape, k, plan, flush=True)
    n, t, h, w, c = shape
    seed = sum(shape) + k + 11
    a = sg.normal(shape, seed, sg.X)
    wt = _w(k, c, seed)
    ci = sg.normal((n, 2, h, w, c), seed, sg.X_PREV)
    b = sg.normal((k,), seed, sg.BETA2, std=0.5, dtype=torch.float32)
    r = sg.normal((n, t, h, w, k), seed, sg.GAMMA2)
    co = torch.empty((n, 2, h, w, c), dtype=torch.bfloat16, device=DEV)
    y = sga.causal_conv3d(a.to(DEV), wt.to(DEV), ci.to(DEV), b.to(DEV), r.to(DEV), cache_out=co)
    torch.cuda.synchronize()
    o, cache_o = oconv.causal_conv3d(vals(a), vals(wt), vals(ci), b.numpy(), vals(r))
    assert_conv_close(bits(y), o, "unfused %s" % (shape,))
    assert np.array_equal(vals(co), cache_o)


def _apply(x, groups, gamma, beta, eps):
    st = sga.gn_silu_stats(x, groups)
    return sga.gn_silu_apply(x, groups, st, gamma, beta, eps), st


def test_latent_block_unfused_two_passes():
    """The latent-resolution block [1,4,44,78,1024] as bench.py runs it (gn_silu_stats,
    gn_silu_apply, then the unfused conv on the 224-row slab tile), two passes: the second
    with the first's cache. Compared in full with the oracle's two passes."""
    wl = WORKLOADS[2]
    assert _plan(wl.shape, wl.k)["tile_m"] == 224
    g, eps = wl.groups, wl.eps
    xp, x = wl.x_prev(), wl.x()
    gamma, beta, wt = wl.gamma(), wl.beta(), wl.conv_weight()
    xpd, xd, gd, bd, wd = (v.to(DEV) for v in (xp, x, gamma, beta, wt))
    print("case latent unfused pass 0", flush=True)
    cache1 = torch.empty((1, 2, wl.h, wl.w, wl.c), dtype=torch.bfloat16, device=DEV)
    ap_gpu, _ = _apply(xpd, g, gd, bd, eps)
    y0 = sga.causal_conv3d(ap_gpu, wd, None, cache_out=cache1)
    print("case latent unfused pass 1", flush=True)
    a_gpu, _ = _apply(xd, g, gd, bd, eps)
    cache2 = torch.empty_like(cache1)
    y = sga.causal_conv3d(a_gpu, wd, cache1, cache_out=cache2)
    torch.cuda.synchronize()
    ap, _ = ogn.gn_silu(vals(xp), g, gamma.numpy(), beta.numpy(), eps)
    act, _ = ogn.gn_silu(vals(x), g, gamma.numpy(), beta.numpy(), eps)
    for name, gpu, o64 in (("act pass 0", ap_gpu, ap), ("act pass 1", a_gpu, act)):
        d = obf16.ulp_distance(bits(gpu), obf16.round_rne(o64))
        assert d.max() <= 1, (name, int(d.max()))
    ap = obf16.decode(obf16.round_rne(ap))
    act = obf16.decode(obf16.round_rne(act))
    o0, oc1 = oconv.causal_conv3d(ap, vals(wt), None)
    o1, oc2 = oconv.causal_conv3d(act, vals(wt), oc1)
    assert_conv_close(bits(y0), o0, "latent pass 0")
    assert_conv_close(bits(y), o1, "latent pass 1")
    # the caches are activated frames: bf16 results of the apply, each within one ulp
    assert obf16.ulp_distance(bits(cache1), obf16.round_rne(oc1)).max() <= 1
    assert obf16.ulp_distance(bits(cache2), obf16.round_rne(oc2)).max() <= 1


def _sampled_conv(src, cache, wt, y, residual=None, bias=None, n_interior=16384, seed=0, what="sampled"):
    """Oracle outputs at sampled positions of a large unfused conv from its (activated) input
    ``src`` and ``cache`` (float32 numpy, exact bf16 values), all K channels each."""
    n, t, h, w, _ = src.shape
    pos = sample_positions(t, h, w, n_interior, seed)
    yb = y.cpu()
    rb = residual.cpu() if residual is not None else None
    wv = vals(wt)
    outs, gots = [], []
    for s in range(0, len(pos), 4096):
        p = pos[s:s + 4096]
        idx = tuple(torch.from_numpy(p[:, i]) for i in range(4))
        o = oconv.conv_at(oconv.causal_patches(src, cache, p), wv, bias)
        if rb is not None:
            o = o + vals(rb[idx])
        outs.append(o)
        gots.append(bits(yb[idx]))
    print("  %d sampled positions" % len(pos), flush=True)
    return assert_conv_close(np.concatenate(gots), np.concatenate(outs), what)


def _sampled_apply(x, act, groups, gamma, beta, eps, stats=None, n_interior=65536, seed=0):
    """GroupNorm+SiLU of ``x`` (float32 numpy) at sampled positions, all channels: the GPU's
    ``act`` within 1 bf16 ulp of the oracle's result rounded once. The oracle's statistics are
    its own, over the whole tensor."""
    n, t, h, w, _ = x.shape
    assert n == 1
    mean, var = ogn.group_stats(x, groups) if stats is None else stats
    pos = sample_positions(t, h, w, n_interior, seed)
    xs = x[pos[:, 0], pos[:, 1], pos[:, 2], pos[:, 3]]
    z = ogn.normalize(xs[None], mean, var, gamma.numpy(), beta.numpy(), eps, groups)[0]
    got = bits(act.cpu()[tuple(torch.from_numpy(pos[:, i]) for i in range(4))])
    d = obf16.ulp_distance(got, obf16.round_rne(ogn.silu(z)))
    print("  apply at %d positions: max ulp %d" % (len(pos), int(d.max())), flush=True)
    assert d.max() <= 1
    return mean, var


@pytest.mark.slow
def test_upsample_block_conv_unfused_sampled():
    """The upsample block's conv 512->512 at [1,8,176,312,512] on the 256 x 256 slab tile:
    GroupNorm+SiLU by gn_silu_apply, then the unfused conv (zero cache)."""
    wl = WORKLOADS[3]
    shape = (1, wl.t, 2 * wl.h, 2 * wl.w, wl.c)
    assert _plan(shape, wl.c) == {"kernel": "slab", "tile_m": 256, "tile_n": 256, "workgroups": 3440}
    x = sg.normal(shape, wl.seed, sg.X_PREV, device=DEV)
    gamma, beta = wl.gamma(), wl.beta()
    wt = sg.normal((wl.c, 3, 3, 3, wl.c), wl.seed, sg.W1, std=1 / math.sqrt(27 * wl.c))
    print("case upsample-block conv, unfused", flush=True)
    act, _ = _apply(x, wl.groups, gamma.to(DEV), beta.to(DEV), wl.eps)
    y = sga.causal_conv3d(act, wt.to(DEV))
    torch.cuda.synchronize()
    _sampled_apply(vals32(x), act, wl.groups, gamma, beta, wl.eps, seed=5)
    _sampled_conv(vals32(act), None, wt, y, seed=6, what="upsample-block conv")


@pytest.mark.slow
def test_fullres_conv_unfused_sampled():
    """One conv of the full-resolution block at [1,16,352,624,256] on the 256 x 256 slab tile,
    with a cache (activated frames of a previous pass) and the residual x."""
    wl = WORKLOADS[4]
    assert _plan(wl.shape, wl.c) == {"kernel": "slab", "tile_m": 256, "tile_n": 256, "workgroups": 13728}
    x = wl.x(device=DEV)
    gamma, beta, wt = wl.gamma(), wl.beta(), wl.conv_weight()
    ci = sg.normal((1, 2, wl.h, wl.w, wl.c), wl.seed, sg.GAMMA2, device=DEV)
    print("case full-res conv, unfused", flush=True)
    act, _ = _apply(x, wl.groups, gamma.to(DEV), beta.to(DEV), wl.eps)
    co = torch.empty_like(ci)
    y = sga.causal_conv3d(act, wt.to(DEV), ci, residual=x, cache_out=co)
    torch.cuda.synchronize()
    assert torch.equal(co.view(torch.int16), act[:, -2:].view(torch.int16))
    _sampled_conv(vals32(act), vals32(ci), wt, y, residual=x, seed=7, what="full-res conv")


@pytest.mark.slow
def test_fullres_block_chain_as_benched():
    """The full-resolution residual block exactly as bench.py's step runs it, over two passes:
    gn_silu_stats + gn_silu_apply of x, conv1 by causal_conv3d_next_stats (norm2's statistics
    from its epilogue), gn_silu_apply of h with those statistics, then conv2 unfused with the
    residual x; each conv with its own cache, carried from a first pass over x_prev.
    Stage-wise against the oracle: norm2's statistics against the oracle's over the GPU's h,
    the applies within 1 ulp at sampled positions, both convs at sampled positions."""
    wl = WORKLOADS[4]
    g, eps = wl.groups, wl.eps
    (g1, b1, w1), (g2, b2, w2) = [(wl.gamma(i), wl.beta(i), wl.conv_weight(i)) for i in (1, 2)]
    g1d, b1d, w1d, g2d, b2d, w2d = (v.to(DEV) for v in (g1, b1, w1, g2, b2, w2))
    shape = wl.shape
    print("case full-res chain pass 0", flush=True)
    xp = wl.x_prev(device=DEV)
    c0 = torch.empty((1, 2, wl.h, wl.w, wl.c), dtype=torch.bfloat16, device=DEV)
    c1 = torch.empty_like(c0)
    a1p, _ = _apply(xp, g, g1d, b1d, eps)
    hp = sga.causal_conv3d(a1p, w1d, None, cache_out=c0)
    a2p, _ = _apply(hp, g, g2d, b2d, eps)
    sga.causal_conv3d(a2p, w2d, None, residual=xp, cache_out=c1)
    del xp, a1p, hp, a2p
    print("case full-res chain pass 1", flush=True)
    x = wl.x(device=DEV)
    a1, _ = _apply(x, g, g1d, b1d, eps)
    h, st2 = sga.causal_conv3d_next_stats(a1, w1d, g, c0)
    a2 = sga.gn_silu_apply(h, g, st2, g2d, b2d, eps)
    y = sga.causal_conv3d(a2, w2d, c1, residual=x)
    torch.cuda.synchronize()
    # norm2's statistics (from conv1's epilogue) against the oracle's over the GPU's h
    hv = vals32(h)
    mean2, var2 = ogn.group_stats(hv, g)
    st2 = st2.cpu().numpy()
    np.testing.assert_allclose(st2[..., 0], mean2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(st2[..., 1], var2, rtol=1e-10, atol=1e-12)
    # the applies, and conv1 / conv2 stage by stage
    xv = vals32(x)
    _sampled_apply(xv, a1, g, g1, b1, eps, seed=8)
    _sampled_apply(hv, a2, g, g2, b2, eps, stats=(mean2, var2), seed=9)
    _sampled_conv(vals32(a1), vals32(c0), w1, h, seed=10, what="chain conv1")
    del hv
    _sampled_conv(vals32(a2), vals32(c1), w2, y, residual=x, seed=11, what="chain conv2 + residual")


@pytest.mark.slow
def test_upsample_block_chain_as_benched():
    """The upsample block exactly as bench.py's step runs it: upsample2x_conv_phases of x
    [1,8,88,156,512], gn_silu_stats + gn_silu_apply of the upsampled u [1,8,176,312,512], then
    the unfused conv (zero cache). Stage-wise against the oracle: the upsample at sampled
    positions against the direct form, the statistics against the oracle's over the GPU's u,
    the apply within 1 ulp and the conv at sampled positions."""
    wl = WORKLOADS[3]
    g, eps = wl.groups, wl.eps
    x = wl.x(device=DEV)
    w3 = wl.up_weight()
    gamma, beta, wt = wl.gamma(), wl.beta(), wl.conv_weight()
    wp = sga.upsample2x_prepare_weights(w3).to(DEV)
    ushape = (1, wl.t, 2 * wl.h, 2 * wl.w, wl.c)
    print("case upsample-block chain", flush=True)
    u = torch.empty(ushape, dtype=torch.bfloat16, device=DEV)
    sga.upsample2x_conv_phases(x, wp, y=u)
    act, st = _apply(u, g, gamma.to(DEV), beta.to(DEV), eps)
    y = sga.causal_conv3d(act, wt.to(DEV))
    torch.cuda.synchronize()
    pos = sample_positions(wl.t, 2 * wl.h, 2 * wl.w, 8192, seed=12)
    idx = tuple(torch.from_numpy(pos[:, i]) for i in range(4))
    o = oconv.upsample2x_conv_at(vals32(x), vals(w3), pos)
    assert_conv_close(bits(u.cpu()[idx]), o, "chain upsample")
    del x
    uv = vals32(u)
    del u
    mean, var = ogn.group_stats(uv, g)
    st = st.cpu().numpy()
    np.testing.assert_allclose(st[..., 0], mean, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(st[..., 1], var, rtol=1e-10, atol=1e-12)
    _sampled_apply(uv, act, g, gamma, beta, eps, stats=(mean, var), seed=13)
    del uv
    _sampled_conv(vals32(act), None, wt, y, seed=14, what="chain conv")

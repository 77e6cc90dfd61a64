"""Causal 3x3x3 convolution on the GPU vs the fp64 oracle (causal_conv3d).

Gate (unit-scale data): relative L2 error <= 1e-2 and max abs error <= 4e-2 against
the unrounded fp64 oracle; the fused GroupNorm variant must equal apply-then-conv
bitwise; cache_out must equal the last 2 frames of the padded input bitwise.
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


def _gn_params(c, seed):
    return (sg.normal((c,), seed, sg.GAMMA1, std=0.1, mean=1.0, dtype=torch.float32),
            sg.normal((c,), seed, sg.BETA1, std=0.1, dtype=torch.float32))


@pytest.mark.parametrize("n,t,h,w,c,k,cache,bias,res", [
    (1, 3, 16, 16, 64, 64, False, False, False),     # the tiny block's shape
    (1, 1, 5, 7, 64, 4, True, True, False),          # T = 1: both taps back into the cache
    (1, 2, 9, 33, 128, 12, True, False, True),       # ragged tiles, K = 12
    (2, 3, 11, 13, 192, 96, True, True, True),       # two samples, K not a tile multiple
    (1, 4, 6, 70, 256, 256, True, True, True),
    pytest.param(1, 2, 7, 9, 512, 520, False, True, False, marks=pytest.mark.skip(
        reason="K past one 256 tile: faulted the GPU once under a since-removed kernel "
               "revision with no cause shown; kept off the GPU until one is")),
    (1, 2, 7, 9, 512, 264, False, True, False),      # K past one 256 tile, ragged
    (1, 2, 3, 4, 4096, 64, True, True, False),       # the largest C: cache rows of 512 packets
    (2, 1, 3, 4, 4096, 128, False, False, True),     # ... without a cache (zeros), two samples
    (1, 2, 3, 5, 64, 4096, True, True, True),        # the largest K: 16 N tiles
    (1, 2, 1, 1, 64, 256, True, True, True),         # a single pixel (slab kernel): 26 of 27 taps padding
    (1, 3, 1, 9, 128, 256, True, False, True),       # one row: the row taps above and below read zeros
    (1, 2, 7, 1, 64, 256, True, True, False),        # one column: every output at both row edges
    (1, 1, 1, 1, 64, 64, False, True, False),        # a single pixel, K <= 128, no cache
    (2, 1, 1, 5, 64, 128, False, False, True),       # one row, T = 1 without a cache, two samples
])
def test_conv_small(n, t, h, w, c, k, cache, bias, res):
    print("case", (n, t, h, w, c, k, cache, bias, res), flush=True)
    seed = n + t + h + w + c + k
    a = sg.normal((n, t, h, w, c), seed, sg.X)
    wt = _w(k, c, seed)
    ci = sg.normal((n, 2, h, w, c), seed, sg.X_PREV) if cache else None
    b = sg.normal((k,), seed, sg.BETA2, std=0.5, dtype=torch.float32) if bias else None
    r = sg.normal((n, t, h, w, k), seed, sg.GAMMA2) if res else None
    co = torch.empty((n, 2, h, w, c), dtype=torch.bfloat16, device=DEV)
    y = sga.causal_conv3d(a.to(DEV), wt.to(DEV), ci.to(DEV) if cache else None,
                          b.to(DEV) if bias else None, r.to(DEV) if res else None, cache_out=co)
    torch.cuda.synchronize()
    o, cache_o = oconv.causal_conv3d(vals(a), vals(wt), vals(ci) if cache else None,
                                     b.numpy() if bias else None, vals(r) if res else None)
    assert_conv_close(bits(y), o, "conv")
    assert np.array_equal(vals(co), cache_o)


def _fused_case(shape, k, groups, seed, cache=True):
    n, t, h, w, c = shape
    x = sg.normal(shape, seed, sg.X, mean=0.2)
    gamma, beta = _gn_params(c, seed)
    wt = _w(k, c, seed)
    ci = sg.normal((n, 2, h, w, c), seed, sg.X_PREV) if cache else None
    return x, gamma, beta, wt, ci


@pytest.mark.parametrize("shape,k,groups", [
    ((1, 3, 16, 16, 64), 64, 32),
    ((2, 1, 7, 9, 256), 32, 32),
    ((1, 3, 5, 37, 1024), 256, 32),
    ((1, 2, 3, 4, 2048), 64, 32),                   # the largest C the fused load takes
    ((1, 2, 1, 1, 64), 64, 32),                     # a single pixel
    ((1, 3, 1, 7, 128), 256, 16),                   # one row, K = 256
])
def test_fused_equals_apply_then_conv_and_oracle(shape, k, groups):
    print("case fused", shape, k, groups, flush=True)
    x, gamma, beta, wt, ci = _fused_case(shape, k, groups, sum(shape) + k)
    xd, gd, bd, wd, cd = (v.to(DEV) for v in (x, gamma, beta, wt, ci))
    eps = 1e-5
    stats = sga.gn_silu_stats(xd, groups)
    a = sga.gn_silu_apply(xd, groups, stats, gd, bd, eps)
    co1 = torch.empty_like(cd)
    co2 = torch.empty_like(cd)
    y1 = sga.causal_conv3d(a, wd, cd, cache_out=co1)
    y2 = sga.causal_conv3d(xd, wd, cd, fuse=(stats, gd, bd, eps, groups), cache_out=co2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(co1.view(torch.int16), co2.view(torch.int16))
    # oracle: GroupNorm+SiLU in fp64, rounded once to bf16, then the conv
    act, st = ogn.gn_silu(vals(x), groups, gamma.numpy(), beta.numpy(), eps)
    act = obf16.decode(obf16.round_rne(act))
    o, cache_o = oconv.causal_conv3d(act, vals(wt), vals(ci))
    assert_conv_close(bits(y2), o, "fused")
    # the cache holds activated frames; they are bf16 results of the same apply
    assert np.array_equal(vals(co2), cache_o) or obf16.ulp_distance(
        bits(co2), obf16.round_rne(cache_o)).max() <= 1


def test_conv_deterministic_causal_and_pass_split():
    n, t, h, w, c, k = 1, 5, 12, 40, 256, 256
    seed = 77
    a = sg.normal((n, t, h, w, c), seed, sg.X).to(DEV)
    wt = _w(k, c, seed).to(DEV)
    c0 = sg.normal((n, 2, h, w, c), seed, sg.X_PREV).to(DEV)
    y = sga.causal_conv3d(a, wt, c0)
    y_again = sga.causal_conv3d(a, wt, c0)
    assert torch.equal(y.view(torch.int16), y_again.view(torch.int16))
    # causality: a change in frame 3 leaves frames 0..2 bitwise unchanged
    b = a.clone()
    b[:, 3] = sg.normal((n, 1, h, w, c), seed, sg.GAMMA2).to(DEV)[:, 0]
    yb = sga.causal_conv3d(b, wt, c0)
    assert torch.equal(yb[:, :3].view(torch.int16), y[:, :3].view(torch.int16))
    assert not torch.equal(yb[:, 3:].view(torch.int16), y[:, 3:].view(torch.int16))
    # pass split: frames [0,2) then [2,5) with the carried cache == one pass
    c1 = torch.empty_like(c0)
    y01 = sga.causal_conv3d(a[:, :2].contiguous(), wt, c0, cache_out=c1)
    y25 = sga.causal_conv3d(a[:, 2:].contiguous(), wt, c1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y01, y25], 1).view(torch.int16), y.view(torch.int16))


def test_latent_block_two_passes():
    """The latent-resolution block [1,4,44,78,1024] with 2 cached frames from a previous pass."""
    wl = WORKLOADS[2]
    g, eps = wl.groups, wl.eps
    xp, x = wl.x_prev(), wl.x()
    gamma, beta, wt = wl.gamma(), wl.beta(), wl.conv_weight()
    xpd, xd, gd, bd, wd = (v.to(DEV) for v in (xp, x, gamma, beta, wt))
    print("case latent pass 0", flush=True)
    cache1 = torch.empty((1, 2, wl.h, wl.w, wl.c), dtype=torch.bfloat16, device=DEV)
    sp = sga.gn_silu_stats(xpd, g)
    sga.causal_conv3d(xpd, wd, None, fuse=(sp, gd, bd, eps, g), cache_out=cache1)
    print("case latent pass 1", flush=True)
    s = sga.gn_silu_stats(xd, g)
    cache2 = torch.empty_like(cache1)
    y = sga.causal_conv3d(xd, wd, cache1, fuse=(s, gd, bd, eps, g), cache_out=cache2)
    torch.cuda.synchronize()
    # oracle: the same two passes
    ap, _ = ogn.gn_silu(vals(xp), g, gamma.numpy(), beta.numpy(), eps)
    ap = obf16.decode(obf16.round_rne(ap))
    _, oc1 = oconv.causal_conv3d(ap, vals(wt), None)
    act, _ = ogn.gn_silu(vals(x), g, gamma.numpy(), beta.numpy(), eps)
    act = obf16.decode(obf16.round_rne(act))
    o, oc2 = oconv.causal_conv3d(act, vals(wt), oc1)
    assert obf16.ulp_distance(bits(cache1), obf16.round_rne(oc1)).max() <= 1
    assert_conv_close(bits(y), o, "latent")


def _sampled_fused_check(x, wt, ci, gamma, beta, groups, eps, y, residual=None, n_interior=16384, seed=0):
    """Oracle at sampled positions of a large fused conv (all K channels each)."""
    n, t, h, w, c = x.shape
    pos = sample_positions(t, h, w, n_interior, seed)
    xv = vals32(x)
    mean, var = ogn.group_stats(xv, groups)
    g64, b64 = gamma.numpy(), beta.numpy()

    def act(v, nidx):
        z = ogn.normalize(v[None], mean, var, g64, b64, eps, groups)[0]
        return obf16.decode(obf16.round_rne(ogn.silu(z)))

    yb = y.cpu()
    civ = vals32(ci) if ci is not None else None
    wv = vals(wt)
    outs, gots = [], []
    for s in range(0, len(pos), 4096):
        p = pos[s:s + 4096]
        idx = tuple(torch.from_numpy(p[:, i]) for i in range(4))
        patches = oconv.causal_patches(xv, civ, p, act=act)
        o = oconv.conv_at(patches, wv)
        if residual is not None:
            o = o + vals(residual[idx])
        outs.append(o)
        gots.append(bits(yb[idx]))
    return assert_conv_close(np.concatenate(gots), np.concatenate(outs), "sampled")


@pytest.mark.slow
def test_upsample_block_conv_full_size_sampled():
    """The 512->512 conv at [1,8,176,312,512] (fused GroupNorm, zero cache), sampled."""
    wl = WORKLOADS[3]
    shape = (1, wl.t, 2 * wl.h, 2 * wl.w, wl.c)
    x = sg.normal(shape, wl.seed, sg.X_PREV, device=DEV)
    gamma, beta, wt = wl.gamma(), wl.beta(), sg.normal((wl.c, 3, 3, 3, wl.c), wl.seed, sg.W1,
                                                       std=1 / math.sqrt(27 * wl.c))
    gd, bd, wd = gamma.to(DEV), beta.to(DEV), wt.to(DEV)
    print("case upsample-block conv", flush=True)
    s = sga.gn_silu_stats(x, wl.groups)
    y = sga.causal_conv3d(x, wd, None, fuse=(s, gd, bd, wl.eps, wl.groups))
    torch.cuda.synchronize()
    _sampled_fused_check(x.cpu(), wt, None, gamma, beta, wl.groups, wl.eps, y, seed=3)


@pytest.mark.slow
def test_fullres_conv_full_size_sampled():
    """One conv of the full-res block at [1,16,352,624,256] with offsets, a cache and a residual."""
    wl = WORKLOADS[4]
    x = wl.x(device=DEV)
    ci = sg.normal((1, 2, wl.h, wl.w, wl.c), wl.seed, sg.GAMMA2, device=DEV)
    gamma, beta, wt = wl.gamma(), wl.beta(), wl.conv_weight()
    gd, bd, wd = gamma.to(DEV), beta.to(DEV), wt.to(DEV)
    print("case full-res conv", flush=True)
    s = sga.gn_silu_stats(x, wl.groups)
    y = sga.causal_conv3d(x, wd, ci, residual=x, fuse=(s, gd, bd, wl.eps, wl.groups))
    torch.cuda.synchronize()
    xc = x.cpu()
    _sampled_fused_check(xc, wt, ci.cpu(), gamma, beta, wl.groups, wl.eps, y, residual=xc, seed=4)


@pytest.mark.parametrize("shape,k,groups,fused,res", [
    ((1, 3, 16, 16, 256), 256, 32, False, True),     # slab kernel, 8 channels per group, residual
    ((1, 2, 5, 37, 256), 1024, 32, False, False),    # four N tiles, 32 channels per group, ragged M
    ((1, 3, 9, 20, 128), 128, 16, False, False),     # conv_kernel (K <= 128)
    ((2, 2, 7, 9, 256), 256, 32, True, False),       # GroupNorm fused in, statistics out, two samples
    ((1, 2, 6, 10, 64), 64, 32, False, False),       # 2 channels per group: the gn_silu_stats route
    ((1, 2, 6, 10, 64), 72, 9, False, False),        # 72 channels in a 128-wide N tile, 9 groups
    ((1, 2, 6, 10, 64), 96, 4, False, False),        # 24 per group, not dividing the N tile: gn_silu_stats
])
def test_conv_next_stats(shape, k, groups, fused, res):
    """causal_conv3d_next_stats: y as causal_conv3d, and GroupNorm statistics of y."""
    print("case next stats", shape, k, groups, fused, res, flush=True)
    n, t, h, w, c = shape
    seed = n + t + h + w + c + k + groups
    x = sg.normal(shape, seed, sg.X, mean=0.1)
    wt = _w(k, c, seed)
    ci = sg.normal((n, 2, h, w, c), seed, sg.X_PREV)
    b = sg.normal((k,), seed, sg.BETA2, std=0.5, dtype=torch.float32)
    r = sg.normal((n, t, h, w, k), seed, sg.GAMMA2) if res else None
    xd, wd, cd, bd = x.to(DEV), wt.to(DEV), ci.to(DEV), b.to(DEV)
    rd = r.to(DEV) if res else None
    fuse, act = None, vals(x)
    if fused:
        gamma, beta = _gn_params(c, seed)
        st_in = sga.gn_silu_stats(xd, 32)
        fuse = (st_in, gamma.to(DEV), beta.to(DEV), 1e-5, 32)
        a64, _ = ogn.gn_silu(vals(x), 32, gamma.numpy(), beta.numpy(), 1e-5)
        act = obf16.decode(obf16.round_rne(a64))
    y1 = sga.causal_conv3d(xd, wd, cd, bd, rd, fuse)
    y2, st = sga.causal_conv3d_next_stats(xd, wd, groups, cd, bd, rd, fuse)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    st = st.cpu().numpy()
    # the same values summed in another fixed order
    ref = sga.gn_silu_stats(y2, groups).cpu().numpy()
    np.testing.assert_allclose(st, ref, rtol=1e-12, atol=1e-14)
    # the oracle: statistics of its convolution rounded once to bf16; y may differ from that
    # rounding by one bf16 ulp in places, which bounds the difference of the statistics
    o, _ = oconv.causal_conv3d(act, vals(wt), vals(ci), b.numpy(), vals(r) if res else None)
    ob = obf16.decode(obf16.round_rne(o))
    mean, var = ogn.group_stats(ob, groups)
    scale = np.sqrt(np.mean(ob.astype(np.float64) ** 2))
    np.testing.assert_allclose(st[..., 0], mean, rtol=0, atol=2.0 ** -7 * scale)
    np.testing.assert_allclose(st[..., 1], var, rtol=2.0 ** -6, atol=2.0 ** -7 * scale * scale)


def test_conv_next_stats_fullres_workload():
    """[1,16,352,624,256] -> K = 256, G = 32 (the full-resolution block's conv1 -> norm2):
    13728 tiles per sample; the epilogue's statistics equal gn_silu_stats over y."""
    wl = WORKLOADS[4]
    print("case next stats full-resolution workload", flush=True)
    x = wl.x(device=DEV)
    wt = wl.conv_weight(1, device=DEV)
    cache = wl.x_prev(device=DEV)[:, -2:].contiguous()
    y, st = sga.causal_conv3d_next_stats(x, wt, wl.groups, cache)
    ref = sga.gn_silu_stats(y, wl.groups)
    torch.cuda.synchronize()
    np.testing.assert_allclose(st.cpu().numpy(), ref.cpu().numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("shape,k,res,store_y,fused", [
    ((1, 2, 5, 7, 64), 256, False, True, False),     # the epilogue applies the norm (one N tile)
    ((1, 3, 17, 19, 128), 256, True, False, False),  # ... y not stored, residual
    ((2, 2, 9, 30, 64), 192, True, True, False),     # ... K = 192: the last wave's channels all past K
    ((1, 2, 3, 5, 64), 128, False, True, False),     # K <= 128: the conv, then rms_silu over y
    ((1, 2, 3, 5, 64), 512, True, True, False),      # two N tiles: the conv, then rms_silu
    ((1, 2, 5, 6, 256), 256, False, True, True),     # GroupNorm fused in: the conv, then rms_silu
])
def test_conv_rms(shape, k, res, store_y, fused):
    """causal_conv3d_rms: y bitwise as causal_conv3d; act within 1 ulp of rms_silu(y) and close
    to the oracle's composition (its conv rounded once, then its RMS norm)."""
    from oracle import rmsnorm as orms
    from oracle import bf16 as obf16
    print("case conv rms", shape, k, res, store_y, fused, flush=True)
    n, t, h, w, c = shape
    seed = n + t + h + w + c + k + 5
    x = sg.normal(shape, seed, sg.X)
    wt = _w(k, c, seed)
    ci = sg.normal((n, 2, h, w, c), seed, sg.X_PREV)
    b = sg.normal((k,), seed, sg.BETA2, std=0.5, dtype=torch.float32)
    r = sg.normal((n, t, h, w, k), seed, sg.GAMMA2) if res else None
    gain = sg.normal((k,), seed, sg.GAMMA1, std=0.2, mean=1.0, dtype=torch.float32)
    xd, wd, cd, bd, gd = (v.to(DEV) for v in (x, wt, ci, b, gain))
    rd = r.to(DEV) if res else None
    fuse = None
    if fused:
        gamma, beta = _gn_params(c, seed)
        fuse = (sga.gn_silu_stats(xd, 32), gamma.to(DEV), beta.to(DEV), 1e-5, 32)
    y, act = sga.causal_conv3d_rms(xd, wd, gd, 1e-6, cd, bd, rd, fuse=fuse, store_y=store_y)
    y_ref = sga.causal_conv3d(xd, wd, cd, bd, rd, fuse=fuse)
    act_ref = sga.rms_silu(y_ref, gd, 1e-6)
    torch.cuda.synchronize()
    if store_y:
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    d = obf16.ulp_distance(bits(act), bits(act_ref))
    print("  act vs rms_silu(y): max ulp %d, exact %.5f" % (d.max(), (d == 0).mean()), flush=True)
    assert d.max() <= 1
    if not fused:
        o, _ = oconv.causal_conv3d(vals(x), vals(wt), vals(ci), b.numpy(), vals(r) if res else None)
        oa = orms.rms_silu(obf16.decode(obf16.round_rne(o)), gain.numpy(), 1e-6)
        assert_conv_close(bits(act), oa, "act vs oracle")


def test_conv_rms_large_tile():
    """[1,16,64,64,64] -> K = 256: 256 tiles of 256 rows fill one wave of the chip, so the
    256 x 256 tile (not the 224-row one) runs the RMS epilogue; y bitwise as causal_conv3d,
    act within 1 ulp of rms_silu(y), with a residual and y stored."""
    shape, k = (1, 16, 64, 64, 64), 256
    seed = 123
    x = sg.normal(shape, seed, sg.X).to(DEV)
    wt = _w(k, 64, seed).to(DEV)
    r = sg.normal(shape[:4] + (k,), seed, sg.GAMMA2).to(DEV)
    gain = sg.normal((k,), seed, sg.GAMMA1, std=0.2, mean=1.0, dtype=torch.float32).to(DEV)
    print("case conv rms large tile", flush=True)
    y, act = sga.causal_conv3d_rms(x, wt, gain, 1e-6, residual=r)
    y_ref = sga.causal_conv3d(x, wt, residual=r)
    act_ref = sga.rms_silu(y_ref, gain, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    d = (act.view(torch.int16).int() - act_ref.view(torch.int16).int()).abs()
    assert int(d.max()) <= 1


@pytest.mark.slow
def test_conv_rms_fullres():
    """The full-resolution conv (C = K = 256 at [1,16,352,624]) with the RMS norm in its
    epilogue and y not stored: act within 1 ulp of rms_silu over causal_conv3d's y."""
    wl = WORKLOADS[4]
    x = wl.x(device=DEV)
    wt = wl.conv_weight(1, DEV)
    gain = wl.gamma(2, DEV)
    print("case conv rms fullres", flush=True)
    _, act = sga.causal_conv3d_rms(x, wt, gain, 1e-6, store_y=False)
    y_ref = sga.causal_conv3d(x, wt)
    act_ref = sga.rms_silu(y_ref, gain, 1e-6)
    torch.cuda.synchronize()
    d = (act.view(torch.int16).int() - act_ref.view(torch.int16).int()).abs()
    print("  max |bit difference| %d, differing %d" % (int(d.max()), int((d > 0).sum())), flush=True)
    assert int(d.max()) <= 1

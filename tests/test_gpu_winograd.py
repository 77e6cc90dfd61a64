"""causal_conv3d_winograd (F(4x4,3x3)) on the GPU against the oracle, stage by stage.

1. The transformed input V the first kernel writes (read back from the workspace) is within
   one bf16 ulp of the oracle's fp64 input transform rounded once.
2. The output is the oracle's Winograd composition (fp64) of the GPU's own bf16 U and V --
   the products and the output transform -- within the conv gate: relL2 <= 1e-2,
   max abs <= 4e-2 (only fp32 accumulation and the one output rounding separate them).
3. The output against the exact fp64 direct convolution (oracle.conv) within the Winograd
   gate derived from the bf16 rounding of U and V:
   - each rounded element carries a relative error of rms eta = 1.66e-3 (one RNE to bf16);
   - for unit-scale i.i.d. data, output pixel (y, x) of a tile then has a relative rms error
     rho_yx = eta sqrt(2 F_y F_x / 9), F_y = sum_a AT[y,a]^2 |B_a|^2 |G_a|^2 = 9.0, 8.6,
     17.3, 94.3 for y = 0..3, i.e. 0.7% at the tile's first pixel and 7.4% (rho_max) at its
     last corner;
   - with the output rounding this predicts relL2 = 2.5e-2 (a bf16 emulation gives 2.4e-2).
   Gate: relL2 <= 4e-2 (1.6x the prediction) and max abs <= 8 rho_max rms(conv output).
cache_out is checked bitwise, and two passes split along T equal one pass bitwise.
"""
import math

import numpy as np
import pytest
import torch

import silu_gn_amd as sga
import synthgen as sg
from oracle import bf16 as obf16
from oracle import conv as oconv
from oracle import winograd as ow
from synthgen.workloads import WORKLOADS
from tests.helpers import assert_conv_close, bits, conv_errors, sample_positions, vals, vals32

pytestmark = pytest.mark.gpu
DEV = "cuda"

WINO_REL_L2 = 4e-2
RHO_MAX = 0.0737


def assert_wino_close(gpu_bits, o64, conv_rms, what=""):
    rel, mx = conv_errors(gpu_bits, o64)
    lim = 8 * RHO_MAX * conv_rms
    print("%s (winograd gate) relL2=%.3e maxabs=%.3e (limit %.3e)" % (what, rel, mx, lim), flush=True)
    assert rel <= WINO_REL_L2 and mx <= lim, (what, rel, mx, lim)
    return rel, mx


def _w(k, c, seed):
    return sg.normal((k, 3, 3, 3, c), seed, sg.W1, std=1 / math.sqrt(27 * c))


def _act(shape, seed, tid=sg.X):
    """Unit-scale activations: SiLU of N(0, 1), rounded to bf16 (the conv's input after its norm)."""
    z = sg.normal(shape, seed, tid, dtype=torch.float32)
    return (z * torch.sigmoid(z)).to(torch.bfloat16)


def _split_ws(ws, n, t, h, w, c, k):
    """(V bf16 [36][N][T+2][TH][TW][C], M fp32 [36][N][T][TH][TW][K]) views of the workspace."""
    th, tw = (h + 3) // 4, (w + 3) // 4
    vb = 36 * n * (t + 2) * th * tw * c * 2
    v = ws[:vb].view(torch.bfloat16).view(36, n, t + 2, th, tw, c)
    mo = (vb + 255) // 256 * 256
    m = ws[mo:mo + 36 * n * t * th * tw * k * 4].view(torch.float32).view(36, n, t, th, tw, k)
    return v, m


@pytest.mark.parametrize("n,t,h,w,c,k,cache,bias,res", [
    (1, 3, 8, 12, 64, 256, True, False, False),     # whole tiles, one N tile
    (2, 2, 7, 9, 128, 264, True, True, True),       # ragged tiles, two N tiles (the second ragged)
    (1, 1, 5, 6, 64, 192, False, True, False),      # T = 1, zero cache, K = 192
    (1, 4, 17, 30, 256, 256, True, True, True),     # several tile rows, ragged
    (1, 2, 1, 1, 64, 256, True, True, True),        # a single pixel: one tile, 15 of its 16 outputs past the frame
    (2, 1, 3, 2, 128, 256, False, True, True),      # less than one tile, T = 1 without a cache
])
def test_winograd_small(n, t, h, w, c, k, cache, bias, res):
    print("case winograd", (n, t, h, w, c, k, cache, bias, res), flush=True)
    seed = n + t + h + w + c + k + 21
    a = _act((n, t, h, w, c), seed)
    wt = _w(k, c, seed)
    ci = _act((n, 2, h, w, c), seed, sg.X_PREV) if cache else None
    b = sg.normal((k,), seed, sg.BETA2, std=0.5, dtype=torch.float32) if bias else None
    r = sg.normal((n, t, h, w, k), seed, sg.GAMMA2) if res else None
    u = sga.winograd_prepare_weights(wt)
    ws = torch.empty(sga.causal_conv3d_winograd_workspace((n, t, h, w, c), k), dtype=torch.uint8, device=DEV)
    co = torch.empty((n, 2, h, w, c), dtype=torch.bfloat16, device=DEV)
    y = sga.causal_conv3d_winograd(a.to(DEV), u.to(DEV), ci.to(DEV) if cache else None,
                                   b.to(DEV) if bias else None, r.to(DEV) if res else None, cache_out=co, ws=ws)
    torch.cuda.synchronize()
    p = oconv.causal_input(vals(a), vals(ci) if cache else None)
    # 1. the transformed input
    v_gpu, m_gpu = _split_ws(ws, n, t, h, w, c, k)
    v_ref = ow.input_transform(p)                                         # (6, 6, N, T+2, TH, TW, C)
    d = obf16.ulp_distance(bits(v_gpu), obf16.round_rne(v_ref.reshape(v_gpu.shape)))
    print("  V: max ulp %d, exact %.5f" % (int(d.max()), float((d == 0).mean())), flush=True)
    assert d.max() <= 1
    # 2. products and output transform of the GPU's own U, V (fp64) against the GPU output
    uv = vals(u).reshape(6, 6, k, 3, c)
    vv = vals(v_gpu).reshape(6, 6, n, t + 2, (h + 3) // 4, (w + 3) // 4, c)
    m = np.zeros((6, 6, n, t) + vv.shape[4:6] + (k,))
    for dt in range(3):
        m += np.einsum("abkc,abntijc->abntijk", uv[:, :, :, dt], vv[:, :, :, dt:dt + t])
    # the products (fp32 on the GPU, fp64 here from the same bf16 operands)
    mg = m_gpu.cpu().double().numpy().reshape(m.shape)
    scale = np.sqrt(np.mean(m ** 2, axis=(2, 3, 4, 5, 6)))                  # per component
    # a component that is exactly zero (inputs all padding, e.g. the first row and column
    # of a one-pixel frame's transform) must be zero on the GPU too
    zero = scale == 0
    assert np.all(mg[zero] == 0)
    err = np.sqrt(np.mean((mg - m) ** 2, axis=(2, 3, 4, 5, 6))) / np.where(zero, 1.0, scale)
    print("  M: worst component rel rms %.3e at %s" % (err.max(), np.unravel_index(err.argmax(), err.shape)),
          flush=True)
    if err.max() > 1e-5:
        a0, b0 = np.unravel_index(err.argmax(), err.shape)
        print("  M[%d,%d] gpu %s vs %s" % (a0, b0, mg[a0, b0].ravel()[:6], m[a0, b0].ravel()[:6]), flush=True)
    assert err.max() <= 1e-5
    comp = ow.output_transform(m)[:, :, :h, :w]
    if bias:
        comp = comp + b.numpy().astype(np.float64)
    if res:
        comp = comp + vals(r)
    assert_conv_close(bits(y), comp, "  output vs Winograd of the GPU's U, V")
    # 3. against the exact direct convolution
    o, cache_o = oconv.causal_conv3d(vals(a), vals(wt), vals(ci) if cache else None,
                                     b.numpy() if bias else None, vals(r) if res else None)
    conv_part = o - (vals(r) if res else 0.0)
    assert_wino_close(bits(y), o, float(np.sqrt(np.mean(conv_part ** 2))), "  output vs direct conv")
    assert np.array_equal(vals(co), cache_o)


def test_winograd_deterministic_and_pass_split():
    n, t, h, w, c, k = 1, 5, 12, 40, 128, 256
    seed = 78
    a = _act((n, t, h, w, c), seed).to(DEV)
    u = sga.winograd_prepare_weights(_w(k, c, seed)).to(DEV)
    c0 = _act((n, 2, h, w, c), seed, sg.X_PREV).to(DEV)
    y = sga.causal_conv3d_winograd(a, u, c0)
    y_again = sga.causal_conv3d_winograd(a, u, c0)
    c1 = torch.empty_like(c0)
    y01 = sga.causal_conv3d_winograd(a[:, :2].contiguous(), u, c0, cache_out=c1)
    y25 = sga.causal_conv3d_winograd(a[:, 2:].contiguous(), u, c1)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_again.view(torch.int16))
    assert torch.equal(torch.cat([y01, y25], 1).view(torch.int16), y.view(torch.int16))


@pytest.mark.slow
def test_winograd_fullres_sampled():
    """The full-resolution block's conv [1,16,352,624,256] -> 256 through Winograd, with a cache
    and the residual x, on the GroupNorm+SiLU output of x; sampled against the exact direct
    convolution (Winograd gate) and the cache bitwise."""
    wl = WORKLOADS[4]
    x = wl.x(device=DEV)
    gamma, beta, wt = wl.gamma().to(DEV), wl.beta().to(DEV), wl.conv_weight()
    st = sga.gn_silu_stats(x, wl.groups)
    act = sga.gn_silu_apply(x, wl.groups, st, gamma, beta, wl.eps)
    ci = _act((1, 2, wl.h, wl.w, wl.c), wl.seed, sg.X_PREV).to(DEV)
    u = sga.winograd_prepare_weights(wt).to(DEV)
    print("case winograd full-res", flush=True)
    co = torch.empty_like(ci)
    y = sga.causal_conv3d_winograd(act, u, ci, residual=x, cache_out=co)
    torch.cuda.synchronize()
    assert torch.equal(co.view(torch.int16), act[:, -2:].view(torch.int16))
    src, cache = vals32(act), vals32(ci)
    pos = sample_positions(wl.t, wl.h, wl.w, 16384, 12)
    yb, xb = y.cpu(), x.cpu()
    wv = vals(wt)
    outs, convs, gots = [], [], []
    for s in range(0, len(pos), 4096):
        pp = pos[s:s + 4096]
        idx = tuple(torch.from_numpy(pp[:, i]) for i in range(4))
        o = oconv.conv_at(oconv.causal_patches(src, cache, pp), wv)
        convs.append(o)
        outs.append(o + vals(xb[idx]))
        gots.append(bits(yb[idx]))
    conv_rms = float(np.sqrt(np.mean(np.concatenate(convs) ** 2)))
    print("  %d sampled positions" % len(pos), flush=True)
    assert_wino_close(np.concatenate(gots), np.concatenate(outs), conv_rms, "full-res winograd")

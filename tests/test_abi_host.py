"""The C ABI on the host: the library loads, exports every declared entry point, and
rejects invalid arguments before enqueuing anything (no GPU needed, no kernel runs).
Every call below is invalid by construction and must come back with an error code."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import silu_gn_amd as sga
from oracle import bf16 as obf16
from oracle import conv as oconv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "silugn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sga.LIB_PATH), reason="libsilugn.so not built")

FAKE = 0x7f0000000000          # 16-byte aligned, never dereferenced: validation fails first
EINVAL, EALIGN, EALIAS, EWORKSPACE = -1, -2, -3, -5


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    lib = sga.load_library()
    names = declared_functions()
    assert set(names) == set(sga.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name


def test_last_error_is_a_string():
    lib = sga.load_library()
    assert isinstance(lib.sgn_last_error(), bytes)


def D(n=1, t=2, h=4, w=4, c=64):
    return sga.sgn_dims(n, t, h, w, c)


def _err(rc, code):
    lib = sga.load_library()
    msg = lib.sgn_last_error().decode()
    assert rc == code, (rc, msg)
    assert msg


def test_eligibility_predicates():
    lib = sga.load_library()
    # GroupNorm: the shapes gn_silu_stats / gn_silu_apply take
    assert lib.gn_silu_eligible(D(c=64), 32) == 1
    assert lib.gn_silu_eligible(D(c=2048), 32) == 1
    assert lib.gn_silu_eligible(D(c=64), 48) == 0            # groups does not divide C
    assert lib.gn_silu_eligible(D(c=96), 8) == 0             # 12 channels per group
    assert lib.gn_silu_eligible(D(c=4096), 32) == 0          # C > 2048
    assert lib.gn_silu_eligible(D(t=0), 32) == 0
    assert lib.sgn_last_error().decode()
    for dims, g in [(D(c=64), 32), (D(c=96), 8), (D(c=4096), 32), (D(c=256), 4)]:
        assert bool(lib.gn_silu_eligible(dims, g)) == (lib.gn_silu_stats_workspace(dims, g) > 0)
    # convolution: shape part of causal_conv3d's checks
    assert lib.causal_conv3d_eligible(D(c=64), 64, 0) == 1
    assert lib.causal_conv3d_eligible(D(c=4096), 4096, 0) == 1
    assert lib.causal_conv3d_eligible(D(c=72), 64, 0) == 0    # C % 64
    assert lib.causal_conv3d_eligible(D(c=64), 6, 0) == 0     # K % 4
    assert lib.causal_conv3d_eligible(D(c=64), 8192, 0) == 0  # K > 4096
    assert lib.causal_conv3d_eligible(D(c=2048), 64, 32) == 1
    assert lib.causal_conv3d_eligible(D(c=4096), 64, 32) == 0  # fused C > 2048
    assert lib.causal_conv3d_eligible(D(c=64), 64, 48) == 0    # fused groups must divide C
    assert lib.causal_conv3d_eligible(sga.sgn_dims(1, 1, 20000, 20000, 64), 64, 0) == 0   # frame > 2 GiB
    assert sga.causal_conv3d_eligible((1, 2, 4, 4, 128), 256) is True


def test_stats_workspace_size():
    lib = sga.load_library()
    assert lib.gn_silu_stats_workspace(D(), 32) > 0
    assert lib.gn_silu_stats_workspace(D(c=60), 32) == 0         # C % 8
    assert lib.gn_silu_stats_workspace(D(c=64), 48) == 0         # groups does not divide C
    assert lib.gn_silu_stats_workspace(D(c=96), 8) == 0          # C/G = 12 not supported
    assert lib.gn_silu_stats_workspace(D(t=0), 32) == 0


def test_stats_rejects():
    lib = sga.load_library()
    _err(lib.gn_silu_stats(FAKE, D(c=64), 48, FAKE, FAKE, 1 << 20, None), EINVAL)
    _err(lib.gn_silu_stats(None, D(), 32, FAKE, FAKE, 1 << 20, None), EINVAL)
    _err(lib.gn_silu_stats(FAKE + 2, D(), 32, FAKE, FAKE, 1 << 20, None), EALIGN)
    _err(lib.gn_silu_stats(FAKE, D(), 32, FAKE, FAKE, 8, None), EWORKSPACE)
    _err(lib.gn_silu_stats(FAKE, D(), 32, FAKE, None, 1 << 20, None), EWORKSPACE)
    _err(lib.gn_silu_stats(FAKE, D(c=4096), 32, FAKE, FAKE, 1 << 30, None), EINVAL)


def test_apply_rejects():
    lib = sga.load_library()
    _err(lib.gn_silu_apply(FAKE, D(), 32, FAKE, FAKE, FAKE, 0.0, FAKE + 4096, None), EINVAL)     # eps
    _err(lib.gn_silu_apply(FAKE, D(), 32, None, FAKE, FAKE, 1e-5, FAKE + 4096, None), EINVAL)
    _err(lib.gn_silu_apply(FAKE, D(), 32, FAKE, FAKE, FAKE, 1e-5, FAKE + 16, None), EALIAS)      # partial overlap
    _err(lib.gn_silu_apply(FAKE, D(), 32, FAKE, FAKE, FAKE, 1e-5, FAKE + 4104, None), EALIGN)


def test_rms_rejects():
    lib = sga.load_library()
    far = FAKE + (1 << 32)
    _err(lib.rms_silu(FAKE, D(c=96), FAKE, 1e-6, far, None), EINVAL)          # C % 64
    _err(lib.rms_silu(FAKE, D(c=8192), FAKE, 1e-6, far, None), EINVAL)        # C > 4096
    _err(lib.rms_silu(FAKE, D(), None, 1e-6, far, None), EINVAL)
    _err(lib.rms_silu(FAKE, D(), FAKE, 0.0, far, None), EINVAL)               # eps
    _err(lib.rms_silu(FAKE, D(), FAKE, float("nan"), far, None), EINVAL)
    _err(lib.rms_silu(FAKE + 8, D(), FAKE, 1e-6, far, None), EALIGN)
    _err(lib.rms_silu(FAKE, D(), FAKE + 2, 1e-6, far, None), EALIGN)
    _err(lib.rms_silu(FAKE, D(), FAKE, 1e-6, FAKE + 16, None), EALIAS)        # partial overlap
    _err(lib.rms_silu(FAKE, D(t=0), FAKE, 1e-6, far, None), EINVAL)


def test_conv_rejects():
    lib = sga.load_library()
    far = FAKE + (1 << 32)
    _err(lib.causal_conv3d(FAKE, D(c=72), None, FAKE + (1 << 30), 64, None, None, None, far, None, None), EINVAL)
    _err(lib.causal_conv3d(FAKE, D(), None, FAKE + (1 << 30), 6, None, None, None, far, None, None), EINVAL)
    _err(lib.causal_conv3d(FAKE, D(), None, None, 64, None, None, None, far, None, None), EINVAL)
    _err(lib.causal_conv3d(FAKE, D(), None, FAKE + (1 << 30), 64, None, None, None, FAKE + 64, None, None), EALIAS)
    _err(lib.causal_conv3d(FAKE, D(), None, FAKE + (1 << 30), 64, None, None, None, far, far + 64, None), EALIAS)
    _err(lib.causal_conv3d(FAKE, D(), None, FAKE + (1 << 30), 64, None, None, None, far + 8, None, None), EALIGN)
    bad = sga.sgn_gn(FAKE, FAKE, FAKE, 1e-5, 48)
    _err(lib.causal_conv3d(FAKE, D(), None, FAKE + (1 << 30), 64, None, None, ctypes.pointer(bad), far, None, None),
         EINVAL)
    bad = sga.sgn_gn(FAKE, FAKE, FAKE, -1.0, 32)
    _err(lib.causal_conv3d(FAKE, D(), None, FAKE + (1 << 30), 64, None, None, ctypes.pointer(bad), far, None, None),
         EINVAL)


def test_conv_rms_rejects():
    lib = sga.load_library()
    far = FAKE + (1 << 32)
    w = FAKE + (1 << 30)
    act = FAKE + (1 << 34)

    def call(k=256, gain=FAKE + (1 << 35), eps=1e-6, y=far, a=act, fuse=None):
        return lib.causal_conv3d_rms(FAKE, D(), None, w, k, None, None, fuse, gain, eps, y, a, None, None)
    _err(call(gain=None), EINVAL)
    _err(call(a=None), EINVAL)
    _err(call(eps=0.0), EINVAL)
    _err(call(k=200), EINVAL)                           # K % 64
    _err(call(k=512, y=None), EINVAL)                   # y may be NULL only in the epilogue form
    _err(call(k=128, y=None), EINVAL)
    _err(call(gain=FAKE + (1 << 35) + 2), EALIGN)
    _err(call(a=act + 8), EALIGN)
    _err(call(a=far + 64), EALIAS)                      # act inside y
    _err(call(a=FAKE + 64), EALIAS)                     # act inside x


def test_rms_input_rejects():
    lib = sga.load_library()
    far = FAKE + (1 << 32)
    w = FAKE + (1 << 30)
    rstd, gain = FAKE + (1 << 35), FAKE + (1 << 36)
    _err(lib.rms_silu_rstd(FAKE, D(c=96), 1e-6, rstd, None), EINVAL)          # C % 64
    _err(lib.rms_silu_rstd(FAKE, D(), 1e-6, None, None), EINVAL)
    _err(lib.rms_silu_rstd(FAKE, D(), 0.0, rstd, None), EINVAL)               # eps
    _err(lib.rms_silu_rstd(FAKE + 8, D(), 1e-6, rstd, None), EALIGN)
    _err(lib.rms_silu_rstd(FAKE, D(), 1e-6, rstd + 4, None), EALIGN)
    _err(lib.rms_silu_rstd(FAKE, D(), 1e-6, FAKE + 64, None), EALIAS)         # rstd inside x

    def call(d=D(), k=64, r=rstd, g=gain, y=far, co=None):
        return lib.causal_conv3d_rms_input(FAKE, d, None, w, k, None, None, r, g, y, co, None)
    _err(call(r=None), EINVAL)
    _err(call(g=None), EINVAL)
    _err(call(d=D(c=4096)), EINVAL)                     # C > 2048 in the operand-load form
    _err(call(k=6), EINVAL)                             # K % 4
    _err(call(r=rstd + 4), EALIGN)
    _err(call(g=gain + 2), EALIGN)
    _err(call(y=rstd), EALIAS)                          # y over rstd
    _err(call(y=FAKE + 64), EALIAS)                     # y inside x


def test_next_stats_workspace_size():
    lib = sga.load_library()
    ws = lib.causal_conv3d_next_stats_workspace(D(), 256, 32)
    assert ws >= lib.gn_silu_stats_workspace(D(c=256), 32) > 0      # covers the gn_silu_stats route
    assert ws >= 1 * 32 * 2 * 2 * 1 * 8                              # and the epilogue's partials
    assert lib.causal_conv3d_next_stats_workspace(D(), 256, 48) == 0  # groups does not divide K
    assert lib.causal_conv3d_next_stats_workspace(D(t=0), 256, 32) == 0


def test_next_stats_rejects():
    lib = sga.load_library()
    far = FAKE + (1 << 32)
    w = FAKE + (1 << 30)
    big = 1 << 30

    def call(k=256, groups=32, stats=far + (1 << 31), ws=far + (1 << 33), ws_bytes=big, y=far):
        return lib.causal_conv3d_next_stats(FAKE, D(), None, w, k, None, None, None, y, None, groups, stats, ws,
                                            ws_bytes, None)
    _err(call(groups=48), EINVAL)                      # groups must divide K
    _err(call(stats=None), EINVAL)
    _err(call(stats=far + (1 << 31) + 4), EALIGN)
    _err(call(ws=None), EWORKSPACE)
    _err(call(ws_bytes=16), EWORKSPACE)
    _err(call(ws=far + (1 << 33) + 8), EALIGN)
    _err(call(ws=far + 64), EALIAS)                    # workspace inside y
    _err(call(k=6, groups=3), EINVAL)                  # the convolution's own checks (K % 4)
    _err(call(k=12, groups=3), EINVAL)                 # y's GroupNorm: K % 8 (gn_silu_stats)
    _err(call(k=96, groups=8), EINVAL)                 # y's GroupNorm: 12 channels per group


def test_upsample_and_head_reject():
    lib = sga.load_library()
    far = FAKE + (1 << 32)
    _err(lib.upsample2x_conv_phases(FAKE, D(c=32), FAKE + (1 << 30), 64, None, far, None), EINVAL)
    _err(lib.upsample2x_conv_phases(FAKE, D(), FAKE + (1 << 30), 64, None, FAKE + 128, None), EALIAS)
    _err(lib.head_conv_d2s(FAKE, D(c=48), None, FAKE + (1 << 30), None, None, 0, far, None, None), EINVAL)
    _err(lib.head_conv_d2s(FAKE, D(), None, FAKE + (1 << 30), None, None, 0, FAKE + 256, None, None), EALIAS)


def test_time_upsample_rejects():
    lib = sga.load_library()
    far = FAKE + (1 << 32)
    w = FAKE + (1 << 30)
    _err(lib.time_upsample_conv(FAKE, D(), None, w, None, 2, far, None, None), EINVAL)           # first
    _err(lib.time_upsample_conv(FAKE, D(c=96), None, w, None, 0, far, None, None), EINVAL)       # C % 64
    _err(lib.time_upsample_conv(FAKE, D(c=4096), None, w, None, 0, far, None, None), EINVAL)     # 2C > 4096
    _err(lib.time_upsample_conv(FAKE, D(), None, None, None, 0, far, None, None), EINVAL)
    _err(lib.time_upsample_conv(FAKE, D(), None, w, None, 0, far + 8, None, None), EALIGN)
    _err(lib.time_upsample_conv(FAKE, D(), None, w, None, 0, FAKE + 64, None, None), EALIAS)     # y inside x
    _err(lib.time_upsample_conv(FAKE, D(), None, w, None, 1, far, far + 64, None), EALIAS)       # cache_out in y


def test_upsample_shortcut_rejects():
    lib = sga.load_library()
    far = FAKE + (1 << 32)
    w = FAKE + (1 << 30)
    src = FAKE + (1 << 34)

    def call(d=D(t=3), k=64, sd=D(t=2), ft=2, first=1, sc=src, y=far):
        return lib.upsample2x_conv_phases_shortcut(FAKE, d, w, k, None, sc, sd, ft, first, y, None)
    _err(call(sc=None), EINVAL)
    _err(call(ft=3), EINVAL)
    _err(call(first=2), EINVAL)
    _err(call(sd=D(t=3)), EINVAL)                   # T = ft T_in - first (ft - 1) = 3 needs T_in = 2
    _err(call(sd=sga.sgn_dims(1, 2, 5, 4, 64)), EINVAL)   # H differs
    _err(call(sd=D(t=2, c=96)), EINVAL)             # C_in must be K or 2K
    _err(call(k=60, sd=D(t=2, c=60)), EINVAL)       # K % 8
    _err(call(sc=src + 8), EALIGN)
    _err(call(y=src + 64), EALIAS)                  # y overlaps the shortcut source
    _err(call(d=D(t=2), sd=D(t=2), ft=1, first=0, y=FAKE + 32), EALIAS)   # the phases' own checks


@pytest.mark.parametrize("k,c", [(4, 8), (16, 64)])
def test_prepare_phase_weights_matches_oracle(k, c):
    w = torch.randn(k, 3, 3, c, generator=torch.Generator().manual_seed(k + c)).to(torch.bfloat16)
    got = sga.upsample2x_prepare_weights(w)
    want = oconv.phase_weights(w.float().numpy().astype(np.float64))     # fp64 sums [a,b,k,u,v,c]
    gb = got.view(torch.int16).numpy().view(np.uint16)
    d = obf16.ulp_distance(gb, obf16.round_rne(want))
    # fp32 sums of at most four bf16 values, rounded once: at most one ulp from the fp64 sum's rounding
    assert d.max() <= 1
    assert (d == 0).mean() > 0.99


def test_prepare_phase_weights_rejects():
    lib = sga.load_library()
    _err(lib.upsample2x_prepare_weights(None, 4, 8, FAKE), EINVAL)
    buf = (ctypes.c_uint16 * (16 * 4 * 8))()
    _err(lib.upsample2x_prepare_weights(ctypes.addressof(buf), 4, 8, ctypes.addressof(buf) + 16), EALIAS)


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_binding_rejects_bad_tensors():
    """The binding checks every tensor before its pointer reaches the library (the C side
    cannot see dtype, strides or shape): wrong dtype, strided views, mis-shaped outputs and
    weights, and tensors on another device raise before any call."""
    x, w = _bf(1, 2, 4, 4, 64), _bf(64, 3, 3, 3, 64)
    with pytest.raises(TypeError, match="x must be torch.bfloat16"):
        sga.causal_conv3d(x.float(), w)
    with pytest.raises(ValueError, match="x must be contiguous"):
        sga.causal_conv3d(_bf(1, 2, 4, 8, 64)[:, :, :, ::2], w)
    with pytest.raises(ValueError, match="y must have shape"):
        sga.causal_conv3d(x, w, y=_bf(1, 2, 4, 4, 32))
    with pytest.raises(ValueError, match="w must have shape"):
        sga.causal_conv3d(x, _bf(64, 3, 3, 3, 32))
    with pytest.raises(TypeError, match="bias must be torch.float32"):
        sga.causal_conv3d(x, w, bias=torch.zeros(64, dtype=torch.float64))
    with pytest.raises(ValueError, match="cache_in must have shape"):
        sga.causal_conv3d(x, w, cache_in=_bf(1, 1, 4, 4, 64))
    with pytest.raises(ValueError, match="residual must be contiguous"):
        sga.causal_conv3d(x, w, residual=_bf(1, 2, 4, 4, 128)[..., ::2])
    with pytest.raises(ValueError, match="fuse stats must have shape"):
        sga.causal_conv3d(x, w, fuse=(torch.zeros(1, 16, 2, dtype=torch.float64), torch.ones(64),
                                      torch.zeros(64), 1e-5, 32))
    with pytest.raises(ValueError, match="x must be a GPU tensor"):
        sga.causal_conv3d(x, w)                                   # every check passed but the device
    with pytest.raises(ValueError, match="stats must have shape"):
        sga.gn_silu_apply(x, 32, torch.zeros(1, 32, 3, dtype=torch.float64), torch.ones(64), torch.zeros(64), 1e-5)
    with pytest.raises(TypeError, match="gamma must be torch.float32"):
        sga.gn_silu_apply(x, 32, torch.zeros(1, 32, 2, dtype=torch.float64), torch.ones(64, dtype=torch.bfloat16),
                          torch.zeros(64), 1e-5)
    with pytest.raises(ValueError, match="y must have shape"):
        sga.rms_silu(x, torch.ones(64), 1e-6, y=_bf(1, 2, 4, 4, 128))
    with pytest.raises(ValueError, match="ws holds"):
        sga.gn_silu_stats(x, 32, ws=torch.empty(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="video must have shape"):
        sga.head_conv_d2s(x, _bf(12, 3, 3, 3, 64), video=_bf(1, 3, 2, 4, 4))
    with pytest.raises(ValueError, match="w_phase must have shape"):
        sga.upsample2x_conv_phases(x, _bf(2, 2, 64, 3, 3, 64))
    with pytest.raises(ValueError, match="shortcut must have shape"):
        sga.upsample2x_conv_phases_shortcut(x, _bf(2, 2, 64, 2, 2, 64), _bf(1, 2, 4, 5, 64), 1, False)
    with pytest.raises(ValueError, match="y must have shape"):
        sga.time_upsample_conv(x, _bf(128, 3, 64), True, y=_bf(1, 4, 4, 4, 64))
    with pytest.raises(TypeError, match="rstd must be torch.float64"):
        sga.causal_conv3d_rms_input(x, w, torch.zeros(1, 2, 4, 4), torch.ones(64))
    with pytest.raises(ValueError, match="rstd must have shape"):
        sga.causal_conv3d_rms_input(x, w, torch.zeros(1, 2, 4, 5, dtype=torch.float64), torch.ones(64))
    with pytest.raises(ValueError, match="gain must have shape"):
        sga.causal_conv3d_rms_input(x, w, torch.zeros(1, 2, 4, 4, dtype=torch.float64), torch.ones(32))
    with pytest.raises(ValueError, match="rstd must have shape"):
        sga.rms_silu_rstd(x, 1e-6, rstd=torch.zeros(1, 2, 4, dtype=torch.float64))
    with pytest.raises(ValueError, match="act must have shape"):
        sga.causal_conv3d_rms(x, w, torch.ones(64), 1e-6, act=_bf(1, 2, 4, 4, 32))
    with pytest.raises(ValueError, match="stats must have shape"):
        sga.causal_conv3d_next_stats(x, w, 32, stats=torch.zeros(1, 16, 2, dtype=torch.float64))
    with pytest.raises(ValueError, match="w3x3 must have shape"):
        sga.upsample2x_prepare_weights(_bf(64, 3, 2, 64))


def test_conv_plan():
    """sgn_conv_plan names the kernel and tile a call would run, and rejects what the call would."""
    p = sga.sgn_conv_plan(sga.SGN_OP_CAUSAL, (1, 16, 352, 624, 256), 256)
    assert p == {"kernel": "slab", "tile_m": 256, "tile_n": 256, "workgroups": 13728}
    assert sga.sgn_conv_plan(sga.SGN_OP_CAUSAL, (1, 4, 44, 78, 1024), 1024)["tile_m"] == 224
    assert sga.sgn_conv_plan(sga.SGN_OP_CAUSAL, (1, 3, 16, 16, 64), 64)["kernel"] == "generic"
    assert sga.sgn_conv_plan(sga.SGN_OP_CAUSAL, (1, 3, 16, 16, 256), 256, fused=True)["kernel"] == "generic"
    assert sga.sgn_conv_plan(sga.SGN_OP_PHASES, (1, 8, 88, 156, 512), 512)["workgroups"] == 3456
    assert sga.sgn_conv_plan(sga.SGN_OP_TIME, (1, 4, 44, 78, 1024), 0)["tile_n"] == 256
    lib = sga.load_library()
    p = sga.sgn_plan()
    _err(lib.sgn_conv_plan(0, D(c=72), 64, 0, ctypes.byref(p)), EINVAL)          # C % 64
    _err(lib.sgn_conv_plan(1, D(), 64, 1, ctypes.byref(p)), EINVAL)               # fused phases
    _err(lib.sgn_conv_plan(7, D(), 64, 0, ctypes.byref(p)), EINVAL)               # unknown op
    _err(lib.sgn_conv_plan(0, D(), 64, 0, None), EINVAL)


def test_stats_and_next_stats_alias_rejects():
    lib = sga.load_library()
    d = D()
    need = lib.gn_silu_stats_workspace(d, 32)
    # the workspace over x, stats over x, stats inside the workspace
    _err(lib.gn_silu_stats(FAKE, d, 32, FAKE + (1 << 24), FAKE + 64, need, None), EALIAS)
    _err(lib.gn_silu_stats(FAKE, d, 32, FAKE + 64, FAKE + (1 << 24), need, None), EALIAS)
    _err(lib.gn_silu_stats(FAKE, d, 32, FAKE + (1 << 24) + 64, FAKE + (1 << 24), need, None), EALIAS)
    nneed = lib.causal_conv3d_next_stats_workspace(d, 64, 32)
    far = FAKE + (1 << 32)
    # ws over x; next_stats over the weights; ws over cache_in (y, next_stats elsewhere)
    _err(lib.causal_conv3d_next_stats(FAKE, d, None, far, 64, None, None, None, far + (1 << 24), None, 32,
                                      far + (2 << 24), FAKE + 1024, nneed, None), EALIAS)
    _err(lib.causal_conv3d_next_stats(FAKE, d, None, far, 64, None, None, None, far + (1 << 24), None, 32,
                                      far + 1024, far + (3 << 24), nneed, None), EALIAS)
    _err(lib.causal_conv3d_next_stats(FAKE, d, far + (4 << 24), far, 64, None, None, None, far + (1 << 24), None,
                                      32, far + (2 << 24), far + (4 << 24) + 512, nneed, None), EALIAS)


def test_noalloc_stats_rejects():
    lib = sga.load_library()
    far = FAKE + (1 << 32)
    _err(lib.gn_silu_stats_noalloc(FAKE, D(c=64), 48, far, None), EINVAL)              # groups
    _err(lib.gn_silu_stats_noalloc(None, D(), 32, far, None), EINVAL)
    _err(lib.gn_silu_stats_noalloc(FAKE + 2, D(), 32, far, None), EALIGN)
    _err(lib.gn_silu_stats_noalloc(FAKE, D(n=200, c=2048), 2048, far, None), EINVAL)   # beyond the scratch
    _err(lib.gn_silu_stats_noalloc(FAKE, D(), 32, FAKE + 64, None), EALIAS)            # stats inside x


@pytest.mark.parametrize("k,c", [(8, 16), (3, 64)])
def test_winograd_weights_match_oracle(k, c):
    """The host F(4x4,3x3) weight prep (fp32 sums, one rounding to bf16) within one bf16 ulp of
    the oracle's fp64 transform rounded once (the fp32 sum may round before the bf16 rounding)."""
    from oracle import winograd as ow
    import synthgen as sg
    w = sg.normal((k, 3, 3, 3, c), k + c, sg.W1, std=0.2)
    u = sga.winograd_prepare_weights(w)
    assert u.shape == (36, k, 3, c)
    ref = ow.weight_transform(w.float().numpy().astype(np.float64))      # (6, 6, K, 3, C)
    ref = obf16.round_rne(ref.reshape(36, k, 3, c))
    got = u.view(torch.int16).numpy().view(np.uint16)
    d = obf16.ulp_distance(got, ref)
    assert d.max() <= 1 and (d == 0).mean() > 0.95


def test_winograd_rejects():
    lib = sga.load_library()
    far = FAKE + (1 << 33)
    ws = far + (1 << 32)
    need = lib.causal_conv3d_winograd_workspace(D(c=64), 256)
    assert need > 0
    assert lib.causal_conv3d_winograd_workspace(D(c=64), 128) == 0                 # K <= 128
    assert lib.causal_conv3d_winograd_workspace(D(c=72), 256) == 0                 # C % 64
    assert lib.causal_conv3d_winograd_workspace(D(t=65534, c=64), 256) == 0        # T + 2 frames per grid
    _err(lib.causal_conv3d_winograd(FAKE, D(), None, far, 120, None, None, far + (1 << 30), None, ws, need, None),
         EINVAL)                                                                      # K % 8, K <= 128
    _err(lib.causal_conv3d_winograd(None, D(), None, far, 256, None, None, far + (1 << 30), None, ws, need, None),
         EINVAL)
    _err(lib.causal_conv3d_winograd(FAKE, D(), None, far, 256, None, None, far + (1 << 30), None, ws, 16, None),
         EWORKSPACE)
    _err(lib.causal_conv3d_winograd(FAKE + 8, D(), None, far, 256, None, None, far + (1 << 30), None, ws, need, None),
         EALIGN)
    _err(lib.causal_conv3d_winograd(FAKE, D(), None, far, 256, None, None, FAKE + 64, None, ws, need, None),
         EALIAS)                                                                      # y inside x
    _err(lib.causal_conv3d_winograd(FAKE, D(), None, far, 256, None, None, far + (1 << 30), None, FAKE + 256, need,
                                    None), EALIAS)                                    # workspace over x
    _err(lib.winograd_prepare_weights(None, 4, 64, FAKE), EINVAL)
    buf = np.zeros(36 * 4 * 3 * 64, dtype=np.uint16)
    _err(lib.winograd_prepare_weights(buf.ctypes.data, 4, 64, buf.ctypes.data + 64), EALIAS)


def test_conv_too_large_for_one_launch():
    """A shape every check admits (4e12 elements) whose tile grid would exceed 2^32 work-items:
    refused on the host with SGN_ELAUNCH before any HIP call (the slab conv's and the head's grids)."""
    lib = sga.load_library()
    d = sga.sgn_dims(1, 62500, 1000, 1000, 64)
    _err(lib.causal_conv3d(FAKE, d, None, FAKE + (1 << 45), 64, None, None, None, FAKE + (1 << 44), None, None),
         -4)
    assert "too large" in lib.sgn_last_error().decode()
    # the head kernel's grid (one workgroup per sample, row pair and 48 columns) likewise
    d = sga.sgn_dims(7000, 1, 2048, 2048, 128)
    _err(lib.head_conv_d2s(FAKE, d, None, FAKE + (1 << 45), None, None, 0, FAKE + (1 << 44), None, None), -4)
    assert "too large" in lib.sgn_last_error().decode()

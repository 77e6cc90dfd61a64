"""Python binding of libsilugn.so (argument marshalling only).

Every function here has the name of the C entry point it calls (see
include/silugn.h) and takes torch tensors for the buffers; the tensors' device
pointers and the current HIP stream are handed to the library, which does all
of the work in its gfx950 kernels. There is no fallback: if the library is not
built, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsilugn.so")

SGN_ERRORS = {-1: "EINVAL", -2: "EALIGN", -3: "EALIAS", -4: "ELAUNCH", -5: "EWORKSPACE"}


class SgnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%s)" % (msg, SGN_ERRORS.get(code, code)))
        self.code = code


class sgn_dims(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("t", ctypes.c_int64), ("h", ctypes.c_int64),
                ("w", ctypes.c_int64), ("c", ctypes.c_int64)]


class sgn_gn(ctypes.Structure):
    _fields_ = [("stats", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("groups", ctypes.c_int)]


EXPORTS = ["sgn_last_error", "gn_silu_eligible", "causal_conv3d_eligible", "gn_silu_stats_workspace", "gn_silu_stats", "gn_silu_apply", "rms_silu",
           "causal_conv3d", "causal_conv3d_rms", "causal_conv3d_next_stats_workspace", "causal_conv3d_next_stats",
           "upsample2x_prepare_weights", "upsample2x_conv_phases", "upsample2x_conv_phases_shortcut",
           "time_upsample_conv", "head_conv_d2s"]

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libsilugn.so (once) and declare its signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libsilugn.so is not built; run `python -m silu_gn_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    gnp = ctypes.POINTER(sgn_gn)
    sigs = {
        "sgn_last_error": (ctypes.c_char_p, []),
        "gn_silu_eligible": (i32, [sgn_dims, i32]),
        "causal_conv3d_eligible": (i32, [sgn_dims, i32, i32]),
        "gn_silu_stats_workspace": (sz, [sgn_dims, i32]),
        "gn_silu_stats": (i32, [vp, sgn_dims, i32, vp, vp, sz, vp]),
        "gn_silu_apply": (i32, [vp, sgn_dims, i32, vp, vp, vp, f32, vp, vp]),
        "rms_silu": (i32, [vp, sgn_dims, vp, f32, vp, vp]),
        "causal_conv3d": (i32, [vp, sgn_dims, vp, vp, i32, vp, vp, gnp, vp, vp, vp]),
        "causal_conv3d_rms": (i32, [vp, sgn_dims, vp, vp, i32, vp, vp, gnp, vp, f32, vp, vp, vp, vp]),
        "causal_conv3d_next_stats_workspace": (sz, [sgn_dims, i32, i32]),
        "causal_conv3d_next_stats": (i32, [vp, sgn_dims, vp, vp, i32, vp, vp, gnp, vp, vp, i32, vp, vp,
                                           sz, vp]),
        "upsample2x_prepare_weights": (i32, [vp, i32, i32, vp]),
        "upsample2x_conv_phases": (i32, [vp, sgn_dims, vp, i32, vp, vp, vp]),
        "upsample2x_conv_phases_shortcut": (i32, [vp, sgn_dims, vp, i32, vp, vp, sgn_dims, i32, i32, vp, vp]),
        "time_upsample_conv": (i32, [vp, sgn_dims, vp, vp, vp, i32, vp, vp, vp]),
        "head_conv_d2s": (i32, [vp, sgn_dims, vp, vp, vp, gnp, i32, vp, vp, vp]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(rc):
    if rc != 0:
        raise SgnError(rc, load_library().sgn_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dims(x):
    n, t, h, w, c = x.shape
    return sgn_dims(n, t, h, w, c)


def _stream(x):
    return torch.cuda.current_stream(x.device).cuda_stream


def _gn(fuse):
    """(stats, gamma, beta, eps, groups) -> sgn_gn pointer, or None."""
    if fuse is None:
        return None, None
    stats, gamma, beta, eps, groups = fuse
    s = sgn_gn(stats.data_ptr(), gamma.data_ptr(), beta.data_ptr(), float(eps), int(groups))
    return ctypes.pointer(s), s


def gn_silu_eligible(dims, groups: int) -> bool:
    return bool(load_library().gn_silu_eligible(sgn_dims(*dims), groups))


def causal_conv3d_eligible(dims, k: int, fuse_groups: int = 0) -> bool:
    return bool(load_library().causal_conv3d_eligible(sgn_dims(*dims), k, fuse_groups))


def gn_silu_stats_workspace(dims, groups: int) -> int:
    return int(load_library().gn_silu_stats_workspace(sgn_dims(*dims), groups))


def gn_silu_stats(x, groups: int, stats=None, ws=None):
    """fp64 [N, G, 2] (mean, biased variance) of bf16 NDHWC ``x``."""
    lib = load_library()
    d = _dims(x)
    if stats is None:
        stats = torch.empty((x.shape[0], groups, 2), dtype=torch.float64, device=x.device)
    need = lib.gn_silu_stats_workspace(d, groups)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib.gn_silu_stats(_ptr(x), d, groups, _ptr(stats), _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(x)))
    return stats


def gn_silu_apply(x, groups: int, stats, gamma, beta, eps: float, y=None):
    """bf16 silu(group_norm(x)); ``y`` may be ``x`` (in place)."""
    lib = load_library()
    if y is None:
        y = torch.empty_like(x)
    _check(lib.gn_silu_apply(_ptr(x), _dims(x), groups, _ptr(stats), _ptr(gamma), _ptr(beta),
                             float(eps), _ptr(y), _stream(x)))
    return y


def rms_silu(x, gain, eps: float, y=None):
    """bf16 silu(rms_norm(x)) per position over the channels; ``y`` may be ``x`` (in place)."""
    lib = load_library()
    if y is None:
        y = torch.empty_like(x)
    _check(lib.rms_silu(_ptr(x), _dims(x), _ptr(gain), float(eps), _ptr(y), _stream(x)))
    return y


def causal_conv3d(x, w, cache_in=None, bias=None, residual=None, fuse=None, y=None, cache_out=None):
    """Causal 3x3x3 conv; ``fuse`` = (stats, gamma, beta, eps, groups) applies GroupNorm+SiLU on load.

    Returns y (bf16 N,T,H,W,K); ``cache_out`` (if given) receives the last 2 frames of the padded input.
    """
    lib = load_library()
    k = w.shape[0]
    if y is None:
        y = torch.empty(x.shape[:4] + (k,), dtype=torch.bfloat16, device=x.device)
    gp, _keep = _gn(fuse)
    _check(lib.causal_conv3d(_ptr(x), _dims(x), _ptr(cache_in), _ptr(w), k, _ptr(bias), _ptr(residual),
                             gp, _ptr(y), _ptr(cache_out), _stream(x)))
    return y


def causal_conv3d_rms(x, w, gain, eps: float, cache_in=None, bias=None, residual=None, fuse=None,
                      y=None, act=None, cache_out=None, store_y=True):
    """causal_conv3d and act = rms_silu(y); returns (y or None, act). ``store_y=False`` skips y
    (allowed when the epilogue applies the norm: unfused, 128 < K <= 256)."""
    lib = load_library()
    k = w.shape[0]
    if y is None and store_y:
        y = torch.empty(x.shape[:4] + (k,), dtype=torch.bfloat16, device=x.device)
    if act is None:
        act = torch.empty(x.shape[:4] + (k,), dtype=torch.bfloat16, device=x.device)
    gp, _keep = _gn(fuse)
    _check(lib.causal_conv3d_rms(_ptr(x), _dims(x), _ptr(cache_in), _ptr(w), k, _ptr(bias), _ptr(residual), gp,
                                 _ptr(gain), float(eps), _ptr(y), _ptr(act), _ptr(cache_out), _stream(x)))
    return y, act


def causal_conv3d_next_stats_workspace(dims, k: int, next_groups: int) -> int:
    return int(load_library().causal_conv3d_next_stats_workspace(sgn_dims(*dims), k, next_groups))


def causal_conv3d_next_stats(x, w, next_groups: int, cache_in=None, bias=None, residual=None, fuse=None,
                             y=None, cache_out=None, stats=None, ws=None):
    """causal_conv3d, plus the GroupNorm statistics (fp64 [N, G, 2]) of its output; returns (y, stats)."""
    lib = load_library()
    k = w.shape[0]
    if y is None:
        y = torch.empty(x.shape[:4] + (k,), dtype=torch.bfloat16, device=x.device)
    if stats is None:
        stats = torch.empty((x.shape[0], next_groups, 2), dtype=torch.float64, device=x.device)
    d = _dims(x)
    need = lib.causal_conv3d_next_stats_workspace(d, k, next_groups)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    gp, _keep = _gn(fuse)
    _check(lib.causal_conv3d_next_stats(_ptr(x), d, _ptr(cache_in), _ptr(w), k, _ptr(bias), _ptr(residual), gp,
                                        _ptr(y), _ptr(cache_out), next_groups, _ptr(stats), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(x)))
    return y, stats


def upsample2x_prepare_weights(w3x3):
    """Host: bf16 (K,3,3,C) -> bf16 phase weights (2,2,K,2,2,C) (CPU tensors)."""
    lib = load_library()
    w = w3x3.detach().to("cpu").contiguous()
    k, _, _, c = w.shape
    out = torch.empty((2, 2, k, 2, 2, c), dtype=torch.bfloat16)
    _check(lib.upsample2x_prepare_weights(w.data_ptr(), k, c, out.data_ptr()))
    return out


def upsample2x_conv_phases(x, w_phase, bias=None, y=None):
    """Nearest-x2 + 3x3 conv via four 2x2 phases; y bf16 (N,T,2H,2W,K)."""
    lib = load_library()
    k = w_phase.shape[2]
    n, t, h, wd, _ = x.shape
    if y is None:
        y = torch.empty((n, t, 2 * h, 2 * wd, k), dtype=torch.bfloat16, device=x.device)
    _check(lib.upsample2x_conv_phases(_ptr(x), _dims(x), _ptr(w_phase), k, _ptr(bias), _ptr(y), _stream(x)))
    return y


def upsample2x_conv_phases_shortcut(x, w_phase, shortcut, ft: int, first: bool, bias=None, y=None):
    """upsample2x_conv_phases plus the DupUp3D shortcut of ``shortcut`` (the block input)."""
    lib = load_library()
    k = w_phase.shape[2]
    n, t, h, wd, _ = x.shape
    if y is None:
        y = torch.empty((n, t, 2 * h, 2 * wd, k), dtype=torch.bfloat16, device=x.device)
    _check(lib.upsample2x_conv_phases_shortcut(_ptr(x), _dims(x), _ptr(w_phase), k, _ptr(bias), _ptr(shortcut),
                                               _dims(shortcut), int(ft), int(bool(first)), _ptr(y), _stream(x)))
    return y


def time_upsample_conv(x, w, first: bool, cache_in=None, bias=None, y=None, cache_out=None):
    """Temporal x2: causal 3x1x1 conv to 2C channels, halves to frames; y (N, first + 2 (T - first), H, W, C)."""
    lib = load_library()
    n, t, h, wd, c = x.shape
    first = int(bool(first))
    if y is None:
        y = torch.empty((n, first + 2 * (t - first), h, wd, c), dtype=torch.bfloat16, device=x.device)
    _check(lib.time_upsample_conv(_ptr(x), _dims(x), _ptr(cache_in), _ptr(w), _ptr(bias), first, _ptr(y),
                                  _ptr(cache_out), _stream(x)))
    return y


def head_conv_d2s(x, w, cache_in=None, bias=None, fuse=None, clamp=False, video=None, cache_out=None):
    """Output head: causal conv to 12 channels + 2x2 depth-to-space; video bf16 (N,3,T,2H,2W)."""
    lib = load_library()
    n, t, h, wd, _ = x.shape
    if video is None:
        video = torch.empty((n, 3, t, 2 * h, 2 * wd), dtype=torch.bfloat16, device=x.device)
    gp, _keep = _gn(fuse)
    _check(lib.head_conv_d2s(_ptr(x), _dims(x), _ptr(cache_in), _ptr(w), _ptr(bias), gp, int(bool(clamp)),
                             _ptr(video), _ptr(cache_out), _stream(x)))
    return video

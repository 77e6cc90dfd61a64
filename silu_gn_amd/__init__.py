"""Python binding of libsilugn.so (argument marshalling only).

Every function here has the name of the C entry point it calls (see
include/silugn.h) and takes torch tensors for the buffers. Each tensor is
checked first (dtype, shape against x and the weights, contiguity, device),
because the C side sees only pointers; then the tensors' device pointers and the
current HIP stream are handed to the library, which does all of the work in
its gfx950 kernels. There is no fallback: if the library is not built, or a
call fails, an exception is raised.
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


class sgn_plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int),
                ("workgroups", ctypes.c_int64)]


SGN_OP_CAUSAL, SGN_OP_PHASES, SGN_OP_TIME = 0, 1, 2
SGN_KERNELS = {1: "slab", 2: "generic"}

EXPORTS = ["sgn_last_error", "gn_silu_eligible", "causal_conv3d_eligible", "sgn_conv_plan", "gn_silu_stats_workspace", "gn_silu_stats", "gn_silu_stats_noalloc", "gn_silu_apply", "rms_silu", "rms_silu_rstd",
           "causal_conv3d", "causal_conv3d_rms", "causal_conv3d_rms_input", "causal_conv3d_next_stats_workspace", "causal_conv3d_next_stats",
           "winograd_prepare_weights", "causal_conv3d_winograd_workspace", "causal_conv3d_winograd",
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
        "sgn_conv_plan": (i32, [i32, sgn_dims, i32, i32, ctypes.POINTER(sgn_plan)]),
        "gn_silu_stats_workspace": (sz, [sgn_dims, i32]),
        "gn_silu_stats": (i32, [vp, sgn_dims, i32, vp, vp, sz, vp]),
        "gn_silu_stats_noalloc": (i32, [vp, sgn_dims, i32, vp, vp]),
        "gn_silu_apply": (i32, [vp, sgn_dims, i32, vp, vp, vp, f32, vp, vp]),
        "rms_silu": (i32, [vp, sgn_dims, vp, f32, vp, vp]),
        "rms_silu_rstd": (i32, [vp, sgn_dims, f32, vp, vp]),
        "causal_conv3d": (i32, [vp, sgn_dims, vp, vp, i32, vp, vp, gnp, vp, vp, vp]),
        "causal_conv3d_rms": (i32, [vp, sgn_dims, vp, vp, i32, vp, vp, gnp, vp, f32, vp, vp, vp, vp]),
        "causal_conv3d_rms_input": (i32, [vp, sgn_dims, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp]),
        "causal_conv3d_next_stats_workspace": (sz, [sgn_dims, i32, i32]),
        "causal_conv3d_next_stats": (i32, [vp, sgn_dims, vp, vp, i32, vp, vp, gnp, vp, vp, i32, vp, vp,
                                           sz, vp]),
        "upsample2x_prepare_weights": (i32, [vp, i32, i32, vp]),
        "winograd_prepare_weights": (i32, [vp, i32, i32, vp]),
        "causal_conv3d_winograd_workspace": (sz, [sgn_dims, i32]),
        "causal_conv3d_winograd": (i32, [vp, sgn_dims, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
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
    """torch's current stream on x's device (the last check before a call: x is on a GPU)."""
    if x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor, got one on %s" % x.device)
    return torch.cuda.current_stream(x.device).cuda_stream


def _arg(t, name, dtype, shape=None, device=None, ndim=None):
    """Check one tensor argument before its pointer reaches the library: the C side sees
    only a pointer, so a wrong dtype, a strided view, a wrong shape or a tensor on another
    device would make it read or write the wrong bytes. ``shape`` entries of None are not
    checked. Raises TypeError (not a tensor, wrong dtype) or ValueError (anything else)."""
    if not torch.is_tensor(t):
        raise TypeError("%s must be a torch tensor, got %s" % (name, type(t).__name__))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, ndim, tuple(t.shape)))
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and s != d for s, d in zip(shape, t.shape)):
            want = "(" + ", ".join("*" if s is None else str(s) for s in shape) + ")"
            raise ValueError("%s must have shape %s, got %s" % (name, want, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (the library reads dense row-major memory)" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    return t


def _act(x, name="x"):
    """A bf16 channels-last activation (N, T, H, W, C): the argument the others follow (their
    device must be x's; that x is on a GPU is checked last, by _stream)."""
    return _arg(x, name, torch.bfloat16, ndim=5)


def _opt(t, name, dtype, shape, device):
    return None if t is None else _arg(t, name, dtype, shape, device)


def _workspace(ws, need, device):
    _arg(ws, "ws", ws.dtype, None, device)
    if ws.numel() * ws.element_size() < need:
        raise ValueError("ws holds %d bytes, %d are needed" % (ws.numel() * ws.element_size(), need))
    return ws


def _gn(fuse, n, c, device):
    """(stats, gamma, beta, eps, groups) -> (sgn_gn pointer, keep-alive), or (None, None)."""
    if fuse is None:
        return None, None
    stats, gamma, beta, eps, groups = fuse
    groups = int(groups)
    _arg(stats, "fuse stats", torch.float64, (n, groups, 2), device)
    _arg(gamma, "fuse gamma", torch.float32, (c,), device)
    _arg(beta, "fuse beta", torch.float32, (c,), device)
    s = sgn_gn(stats.data_ptr(), gamma.data_ptr(), beta.data_ptr(), float(eps), groups)
    return ctypes.pointer(s), s


def gn_silu_eligible(dims, groups: int) -> bool:
    return bool(load_library().gn_silu_eligible(sgn_dims(*dims), groups))


def causal_conv3d_eligible(dims, k: int, fuse_groups: int = 0) -> bool:
    return bool(load_library().causal_conv3d_eligible(sgn_dims(*dims), k, fuse_groups))


def sgn_conv_plan(op: int, dims, k: int, fused: bool = False) -> dict:
    """The kernel ("slab" / "generic"), tile and workgroup count a convolution call would run."""
    p = sgn_plan()
    _check(load_library().sgn_conv_plan(int(op), sgn_dims(*dims), int(k), int(bool(fused)), ctypes.byref(p)))
    return {"kernel": SGN_KERNELS[p.kernel], "tile_m": p.tile_m, "tile_n": p.tile_n, "workgroups": p.workgroups}


def gn_silu_stats_workspace(dims, groups: int) -> int:
    return int(load_library().gn_silu_stats_workspace(sgn_dims(*dims), groups))


def gn_silu_stats(x, groups: int, stats=None, ws=None):
    """fp64 [N, G, 2] (mean, biased variance) of bf16 NDHWC ``x``."""
    lib = load_library()
    _act(x)
    d, dev, groups = _dims(x), x.device, int(groups)
    need = lib.gn_silu_stats_workspace(d, groups)
    if stats is None:
        stats = torch.empty((x.shape[0], groups, 2), dtype=torch.float64, device=dev)
    _arg(stats, "stats", torch.float64, (x.shape[0], groups, 2), dev)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _workspace(ws, need, dev)
    _check(lib.gn_silu_stats(_ptr(x), d, groups, _ptr(stats), _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(x)))
    return stats


def gn_silu_stats_noalloc(x, groups: int, stats):
    """gn_silu_stats with no workspace: the library's static scratch holds the partial sums."""
    lib = load_library()
    _act(x)
    _arg(stats, "stats", torch.float64, (x.shape[0], int(groups), 2), x.device)
    _check(lib.gn_silu_stats_noalloc(_ptr(x), _dims(x), int(groups), _ptr(stats), _stream(x)))
    return stats


def gn_silu_apply(x, groups: int, stats, gamma, beta, eps: float, y=None):
    """bf16 silu(group_norm(x)); ``y`` may be ``x`` (in place)."""
    lib = load_library()
    _act(x)
    dev, (n, c), groups = x.device, (x.shape[0], x.shape[4]), int(groups)
    _arg(stats, "stats", torch.float64, (n, groups, 2), dev)
    _arg(gamma, "gamma", torch.float32, (c,), dev)
    _arg(beta, "beta", torch.float32, (c,), dev)
    if y is None:
        y = torch.empty_like(x)
    _arg(y, "y", torch.bfloat16, tuple(x.shape), dev)
    _check(lib.gn_silu_apply(_ptr(x), _dims(x), groups, _ptr(stats), _ptr(gamma), _ptr(beta),
                             float(eps), _ptr(y), _stream(x)))
    return y


def rms_silu(x, gain, eps: float, y=None):
    """bf16 silu(rms_norm(x)) per position over the channels; ``y`` may be ``x`` (in place)."""
    lib = load_library()
    _act(x)
    _arg(gain, "gain", torch.float32, (x.shape[4],), x.device)
    if y is None:
        y = torch.empty_like(x)
    _arg(y, "y", torch.bfloat16, tuple(x.shape), x.device)
    _check(lib.rms_silu(_ptr(x), _dims(x), _ptr(gain), float(eps), _ptr(y), _stream(x)))
    return y


def rms_silu_rstd(x, eps: float, rstd=None):
    """fp64 [N, T, H, W]: each position's 1 / sqrt(mean_c x^2 + eps), the factor rms_silu applies."""
    lib = load_library()
    _act(x)
    if rstd is None:
        rstd = torch.empty(tuple(x.shape[:4]), dtype=torch.float64, device=x.device)
    _arg(rstd, "rstd", torch.float64, tuple(x.shape[:4]), x.device)
    _check(lib.rms_silu_rstd(_ptr(x), _dims(x), float(eps), _ptr(rstd), _stream(x)))
    return rstd


def _conv_args(x, w, cache_in, bias, residual, y, cache_out, k=None):
    """Checks shared by the causal convolutions; returns (K, y)."""
    _act(x)
    n, t, h, wd, c = x.shape
    dev = x.device
    _arg(w, "w", torch.bfloat16, (k, 3, 3, 3, c), dev)
    k = w.shape[0]
    _opt(cache_in, "cache_in", torch.bfloat16, (n, 2, h, wd, c), dev)
    _opt(bias, "bias", torch.float32, (k,), dev)
    _opt(residual, "residual", torch.bfloat16, (n, t, h, wd, k), dev)
    _opt(cache_out, "cache_out", torch.bfloat16, (n, 2, h, wd, c), dev)
    _opt(y, "y", torch.bfloat16, (n, t, h, wd, k), dev)
    return k


def causal_conv3d(x, w, cache_in=None, bias=None, residual=None, fuse=None, y=None, cache_out=None):
    """Causal 3x3x3 conv; ``fuse`` = (stats, gamma, beta, eps, groups) applies GroupNorm+SiLU on load.

    Returns y (bf16 N,T,H,W,K); ``cache_out`` (if given) receives the last 2 frames of the padded input.
    """
    lib = load_library()
    k = _conv_args(x, w, cache_in, bias, residual, y, cache_out)
    gp, _keep = _gn(fuse, x.shape[0], x.shape[4], x.device)
    if y is None:
        y = torch.empty(x.shape[:4] + (k,), dtype=torch.bfloat16, device=x.device)
    _check(lib.causal_conv3d(_ptr(x), _dims(x), _ptr(cache_in), _ptr(w), k, _ptr(bias), _ptr(residual),
                             gp, _ptr(y), _ptr(cache_out), _stream(x)))
    return y


def causal_conv3d_rms(x, w, gain, eps: float, cache_in=None, bias=None, residual=None, fuse=None,
                      y=None, act=None, cache_out=None, store_y=True):
    """causal_conv3d and act = rms_silu(y); returns (y or None, act). ``store_y=False`` skips y
    (allowed when the epilogue applies the norm: unfused, 128 < K <= 256)."""
    lib = load_library()
    k = _conv_args(x, w, cache_in, bias, residual, y, cache_out)
    _arg(gain, "gain", torch.float32, (k,), x.device)
    _opt(act, "act", torch.bfloat16, tuple(x.shape[:4]) + (k,), x.device)
    gp, _keep = _gn(fuse, x.shape[0], x.shape[4], x.device)
    if y is None and store_y:
        y = torch.empty(x.shape[:4] + (k,), dtype=torch.bfloat16, device=x.device)
    if act is None:
        act = torch.empty(x.shape[:4] + (k,), dtype=torch.bfloat16, device=x.device)
    _check(lib.causal_conv3d_rms(_ptr(x), _dims(x), _ptr(cache_in), _ptr(w), k, _ptr(bias), _ptr(residual), gp,
                                 _ptr(gain), float(eps), _ptr(y), _ptr(act), _ptr(cache_out), _stream(x)))
    return y, act


def causal_conv3d_rms_input(x, w, rstd, gain, cache_in=None, bias=None, residual=None, y=None, cache_out=None):
    """causal_conv3d of rms_silu(x, gain) with the norm applied as the rows of x load; ``rstd`` from
    rms_silu_rstd(x, eps). Returns y; ``cache_out`` (if given) receives the activated last 2 frames."""
    lib = load_library()
    k = _conv_args(x, w, cache_in, bias, residual, y, cache_out)
    _arg(rstd, "rstd", torch.float64, tuple(x.shape[:4]), x.device)
    _arg(gain, "gain", torch.float32, (x.shape[4],), x.device)
    if y is None:
        y = torch.empty(x.shape[:4] + (k,), dtype=torch.bfloat16, device=x.device)
    _check(lib.causal_conv3d_rms_input(_ptr(x), _dims(x), _ptr(cache_in), _ptr(w), k, _ptr(bias), _ptr(residual),
                                       _ptr(rstd), _ptr(gain), _ptr(y), _ptr(cache_out), _stream(x)))
    return y


def causal_conv3d_next_stats_workspace(dims, k: int, next_groups: int) -> int:
    return int(load_library().causal_conv3d_next_stats_workspace(sgn_dims(*dims), k, next_groups))


def causal_conv3d_next_stats(x, w, next_groups: int, cache_in=None, bias=None, residual=None, fuse=None,
                             y=None, cache_out=None, stats=None, ws=None):
    """causal_conv3d, plus the GroupNorm statistics (fp64 [N, G, 2]) of its output; returns (y, stats)."""
    lib = load_library()
    k = _conv_args(x, w, cache_in, bias, residual, y, cache_out)
    gp, _keep = _gn(fuse, x.shape[0], x.shape[4], x.device)
    next_groups = int(next_groups)
    d, dev = _dims(x), x.device
    need = lib.causal_conv3d_next_stats_workspace(d, k, next_groups)
    if y is None:
        y = torch.empty(x.shape[:4] + (k,), dtype=torch.bfloat16, device=dev)
    if stats is None:
        stats = torch.empty((x.shape[0], next_groups, 2), dtype=torch.float64, device=dev)
    _arg(stats, "stats", torch.float64, (x.shape[0], next_groups, 2), dev)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _workspace(ws, need, dev)
    _check(lib.causal_conv3d_next_stats(_ptr(x), d, _ptr(cache_in), _ptr(w), k, _ptr(bias), _ptr(residual), gp,
                                        _ptr(y), _ptr(cache_out), next_groups, _ptr(stats), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(x)))
    return y, stats


def upsample2x_prepare_weights(w3x3):
    """Host: bf16 (K,3,3,C) -> bf16 phase weights (2,2,K,2,2,C) (CPU tensors)."""
    lib = load_library()
    w = w3x3.detach().to("cpu").contiguous()
    _arg(w, "w3x3", torch.bfloat16, (None, 3, 3, None))
    k, _, _, c = w.shape
    out = torch.empty((2, 2, k, 2, 2, c), dtype=torch.bfloat16)
    _check(lib.upsample2x_prepare_weights(w.data_ptr(), k, c, out.data_ptr()))
    return out


def winograd_prepare_weights(w):
    """Host: bf16 (K,3,3,3,C) -> bf16 F(4x4,3x3) weights (36,K,3,C) (CPU tensors)."""
    lib = load_library()
    w = w.detach().to("cpu").contiguous()
    _arg(w, "w", torch.bfloat16, (None, 3, 3, 3, None))
    k, c = w.shape[0], w.shape[4]
    out = torch.empty((36, k, 3, c), dtype=torch.bfloat16)
    _check(lib.winograd_prepare_weights(w.data_ptr(), k, c, out.data_ptr()))
    return out


def causal_conv3d_winograd_workspace(dims, k: int) -> int:
    return int(load_library().causal_conv3d_winograd_workspace(sgn_dims(*dims), int(k)))


def causal_conv3d_winograd(x, u, cache_in=None, bias=None, residual=None, y=None, cache_out=None, ws=None):
    """causal_conv3d through Winograd F(4x4,3x3) with the weights of winograd_prepare_weights (on the
    device); returns y. ``ws`` receives the transformed input and the products (see the header)."""
    lib = load_library()
    _act(x)
    n, t, h, wd, c = x.shape
    dev = x.device
    _arg(u, "u", torch.bfloat16, (36, None, 3, c), dev)
    k = u.shape[1]
    _opt(cache_in, "cache_in", torch.bfloat16, (n, 2, h, wd, c), dev)
    _opt(bias, "bias", torch.float32, (k,), dev)
    _opt(residual, "residual", torch.bfloat16, (n, t, h, wd, k), dev)
    _opt(cache_out, "cache_out", torch.bfloat16, (n, 2, h, wd, c), dev)
    d = _dims(x)
    need = lib.causal_conv3d_winograd_workspace(d, k)
    if need == 0:
        _check(-1)
    if y is None:
        y = torch.empty((n, t, h, wd, k), dtype=torch.bfloat16, device=dev)
    _arg(y, "y", torch.bfloat16, (n, t, h, wd, k), dev)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _workspace(ws, need, dev)
    _check(lib.causal_conv3d_winograd(_ptr(x), d, _ptr(cache_in), _ptr(u), k, _ptr(bias), _ptr(residual),
                                      _ptr(y), _ptr(cache_out), _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(x)))
    return y


def _phase_args(x, w_phase, bias, y):
    _act(x)
    n, t, h, wd, c = x.shape
    _arg(w_phase, "w_phase", torch.bfloat16, (2, 2, None, 2, 2, c), x.device)
    k = w_phase.shape[2]
    _opt(bias, "bias", torch.float32, (k,), x.device)
    _opt(y, "y", torch.bfloat16, (n, t, 2 * h, 2 * wd, k), x.device)
    return k


def upsample2x_conv_phases(x, w_phase, bias=None, y=None):
    """Nearest-x2 + 3x3 conv via four 2x2 phases; y bf16 (N,T,2H,2W,K)."""
    lib = load_library()
    k = _phase_args(x, w_phase, bias, y)
    n, t, h, wd, _ = x.shape
    if y is None:
        y = torch.empty((n, t, 2 * h, 2 * wd, k), dtype=torch.bfloat16, device=x.device)
    _check(lib.upsample2x_conv_phases(_ptr(x), _dims(x), _ptr(w_phase), k, _ptr(bias), _ptr(y), _stream(x)))
    return y


def upsample2x_conv_phases_shortcut(x, w_phase, shortcut, ft: int, first: bool, bias=None, y=None):
    """upsample2x_conv_phases plus the DupUp3D shortcut of ``shortcut`` (the block input)."""
    lib = load_library()
    k = _phase_args(x, w_phase, bias, y)
    n, t, h, wd, _ = x.shape
    _arg(shortcut, "shortcut", torch.bfloat16, (n, None, h, wd, None), x.device)
    if y is None:
        y = torch.empty((n, t, 2 * h, 2 * wd, k), dtype=torch.bfloat16, device=x.device)
    _check(lib.upsample2x_conv_phases_shortcut(_ptr(x), _dims(x), _ptr(w_phase), k, _ptr(bias), _ptr(shortcut),
                                               _dims(shortcut), int(ft), int(bool(first)), _ptr(y), _stream(x)))
    return y


def time_upsample_conv(x, w, first: bool, cache_in=None, bias=None, y=None, cache_out=None):
    """Temporal x2: causal 3x1x1 conv to 2C channels, halves to frames; y (N, first + 2 (T - first), H, W, C)."""
    lib = load_library()
    _act(x)
    n, t, h, wd, c = x.shape
    dev = x.device
    first = int(bool(first))
    _arg(w, "w", torch.bfloat16, (2 * c, 3, c), dev)
    _opt(cache_in, "cache_in", torch.bfloat16, (n, 2, h, wd, c), dev)
    _opt(bias, "bias", torch.float32, (2 * c,), dev)
    _opt(cache_out, "cache_out", torch.bfloat16, (n, 2, h, wd, c), dev)
    to = first + 2 * (t - first)
    if y is None:
        y = torch.empty((n, to, h, wd, c), dtype=torch.bfloat16, device=dev)
    _arg(y, "y", torch.bfloat16, (n, to, h, wd, c), dev)
    _check(lib.time_upsample_conv(_ptr(x), _dims(x), _ptr(cache_in), _ptr(w), _ptr(bias), first, _ptr(y),
                                  _ptr(cache_out), _stream(x)))
    return y


def head_conv_d2s(x, w, cache_in=None, bias=None, fuse=None, clamp=False, video=None, cache_out=None):
    """Output head: causal conv to 12 channels + 2x2 depth-to-space; video bf16 (N,3,T,2H,2W)."""
    lib = load_library()
    _conv_args(x, w, cache_in, bias, None, None, cache_out, k=12)
    n, t, h, wd, _ = x.shape
    gp, _keep = _gn(fuse, n, x.shape[4], x.device)
    if video is None:
        video = torch.empty((n, 3, t, 2 * h, 2 * wd), dtype=torch.bfloat16, device=x.device)
    _arg(video, "video", torch.bfloat16, (n, 3, t, 2 * h, 2 * wd), x.device)
    _check(lib.head_conv_d2s(_ptr(x), _dims(x), _ptr(cache_in), _ptr(w), _ptr(bias), gp, int(bool(clamp)),
                             _ptr(video), _ptr(cache_out), _stream(x)))
    return video

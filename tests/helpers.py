"""Shared test helpers: tensor <-> numpy, parity metrics, sampled positions."""
from __future__ import annotations

import numpy as np
import torch

from oracle import bf16 as obf16


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def vals(t: torch.Tensor) -> np.ndarray:
    """bf16/fp32 tensor (any device) -> exact float64 numpy values."""
    return t.detach().to("cpu").float().numpy().astype(np.float64)


def vals32(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> exact float32 numpy values (half the memory of float64 for big tensors)."""
    return t.detach().to("cpu").float().numpy()


def ulp_report(gpu_bits: np.ndarray, o64: np.ndarray):
    """(max ulp distance, fraction of exact matches) of GPU bf16 vs RNE_bf16(oracle fp64)."""
    ref = obf16.round_rne(o64)
    d = obf16.ulp_distance(gpu_bits, ref)
    return int(d.max()) if d.size else 0, float((d == 0).mean()) if d.size else 1.0


def conv_errors(gpu_bits: np.ndarray, o64: np.ndarray):
    """(relative L2 error, max abs error) of GPU bf16 vs the unrounded fp64 oracle."""
    g = obf16.decode(gpu_bits)
    diff = g - o64
    rel = float(np.linalg.norm(diff.ravel()) / max(np.linalg.norm(o64.ravel()), 1e-300))
    return rel, float(np.abs(diff).max()) if diff.size else 0.0


REL_L2 = 1e-2      # conv tolerances on unit-scale data
MAX_ABS = 4e-2


def assert_conv_close(gpu_bits, o64, what=""):
    rel, mx = conv_errors(gpu_bits, o64)
    print("%s relL2=%.3e maxabs=%.3e" % (what, rel, mx), flush=True)
    assert rel <= REL_L2 and mx <= MAX_ABS, (what, rel, mx)
    return rel, mx


def sample_positions(t, h, w, n_interior, seed, frames=None, n=0):
    """Every border position of frames {0, 1, T-1} plus seeded interior positions: (S, 4) of (n, t, h, w)."""
    frames = sorted(set([0, min(1, t - 1), t - 1])) if frames is None else frames
    pos = []
    for f in frames:
        for x in range(w):
            pos.append((n, f, 0, x))
            pos.append((n, f, h - 1, x))
        for y in range(1, h - 1):
            pos.append((n, f, y, 0))
            pos.append((n, f, y, w - 1))
    rng = np.random.default_rng(seed)
    inner = np.stack([np.full(n_interior, n), rng.integers(0, t, n_interior),
                      rng.integers(0, h, n_interior), rng.integers(0, w, n_interior)], axis=1)
    allpos = np.concatenate([np.array(pos, dtype=np.int64).reshape(-1, 4), inner.astype(np.int64)])
    return np.unique(allpos, axis=0)

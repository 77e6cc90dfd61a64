"""RMS norm + SiLU per position, the plain definition in float64 (test infrastructure only).

The decoder on the FastVideo pages ("wan22_vae_decode binding.cpp", the comment above
Decoder::output_head) normalises with an RMS norm followed by SiLU, with a per-channel
gain (norm_pad(x, gain, ...)). The pages do not print the formula; the reading used
here is the usual RMS norm over the channels of one position:

    z[p, c] = x[p, c] * gain[c] / sqrt(mean_c(x[p, :]^2) + eps)
    out[p, c] = z * sigmoid(z)

computed in float64 and rounded once by the caller. Unlike GroupNorm there are no
statistics across positions: every position (n, t, h, w) is normalised on its own, so a
pass split of the video changes nothing.

Layout: channels-last (..., C); gain has C entries.
"""
from __future__ import annotations

import numpy as np

from oracle.groupnorm import silu


def rms_silu(x, gain, eps: float):
    """float64 silu(rms_norm(x)) over the last axis; x holds exact bf16 values (any float dtype)."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gain, dtype=np.float64)
    assert x.shape[-1] == g.shape[0]
    ms = np.mean(x * x, axis=-1, keepdims=True)          # mean of squares over the channels
    z = x * g / np.sqrt(ms + eps)
    return silu(z)


def rms_rstd(x, eps: float):
    """float64 1 / sqrt(mean_c(x^2) + eps) per position (the factor rms_silu applies with the
    gain): shape x.shape[:-1]. x holds exact bf16 values (any float dtype)."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)

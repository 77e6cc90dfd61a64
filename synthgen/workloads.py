"""The five synthetic workloads: shapes, seeds and value distributions.

Shapes follow the Wan2.2-style VAE decoder of the pages (binding.cpp: latent
grid 44x78 with 4 latent frames per pass; up blocks at 88x156 and 176x312; the
pixel plane 352x624 feeding the output head that writes a 704x1248 video).
Activations are channels-last (N, T, H, W, C) bf16; convolution weights are
(K, kt, kh, kw, C) bf16; GroupNorm affine parameters and conv biases are fp32.

Recipe (one seed per workload, tensor ids from ``synthgen``):
  * activations ~ N(0, 1) rounded once to bf16 (the full-res block adds a
    per-channel offset U(-4, 4) before the rounding);
  * GroupNorm gamma ~ 1 + 0.1 N(0, 1), beta ~ 0.1 N(0, 1), fp32;
  * conv weights ~ N(0, 1 / (taps * C)) read as a variance, drawn in float64 and
    rounded once to bf16; conv bias 0.
Nothing here computes any part of the method.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

import synthgen as sg


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    seed: int
    n: int
    c: int
    t: int
    h: int
    w: int
    k: int
    groups: int = 32
    eps: float = 1e-5
    kind: str = "block"        # block | latent | upsample | resblock | head
    cache_from_prev: bool = False
    channel_offsets: bool = False

    @property
    def shape(self):
        return (self.n, self.t, self.h, self.w, self.c)

    @property
    def numel(self):
        return math.prod(self.shape)

    def x(self, device="cpu", frames=None):
        """The input; ``frames``: only its first frames (drawn alone: the generator is
        counter-based, so they equal the whole tensor's first frames; N = 1 only)."""
        mean = self.offsets(device) if self.channel_offsets else 0.0
        shape = self.shape
        if frames is not None:
            assert self.n == 1 and 1 <= frames <= self.t
            shape = (1, frames) + shape[2:]
        return sg.normal(shape, self.seed, sg.X, mean=mean, device=device)

    def x_prev(self, device="cpu"):
        mean = self.offsets(device) if self.channel_offsets else 0.0
        return sg.normal(self.shape, self.seed, sg.X_PREV, mean=mean, device=device)

    def offsets(self, device="cpu"):
        return sg.uniform((self.c,), self.seed, sg.OFFSETS, -4.0, 4.0, dtype=torch.float32, device=device)

    def gamma(self, which=1, device="cpu"):
        tid = sg.GAMMA1 if which == 1 else sg.GAMMA2
        return sg.normal((self.c,), self.seed, tid, std=0.1, mean=1.0, dtype=torch.float32, device=device)

    def beta(self, which=1, device="cpu"):
        tid = sg.BETA1 if which == 1 else sg.BETA2
        return sg.normal((self.c,), self.seed, tid, std=0.1, dtype=torch.float32, device=device)

    def conv_weight(self, which=1, device="cpu", k=None):
        k = self.k if k is None else k
        tid = sg.W1 if which == 1 else sg.W2
        std = 1.0 / math.sqrt(27 * self.c)
        return sg.normal((k, 3, 3, 3, self.c), self.seed, tid, std=std, device=device)

    def up_weight(self, device="cpu"):
        """The 3x3 spatial weight of the nearest-x2 upsampler, (K, 3, 3, C), K = C."""
        std = 1.0 / math.sqrt(9 * self.c)
        return sg.normal((self.c, 3, 3, self.c), self.seed, sg.W_UP, std=std, device=device)

    def scaled(self, t=None, h=None, w=None, c=None, k=None):
        """The same recipe at a smaller shape (for oracle-sized parity runs)."""
        from dataclasses import replace
        return replace(self, t=t or self.t, h=h or self.h, w=w or self.w,
                       c=c or self.c, k=k or self.k)


WORKLOADS = {
    1: Workload(1, "tiny_block", 0, 1, 64, 3, 16, 16, 64, kind="block"),
    2: Workload(2, "latent_block", 1, 1, 1024, 4, 44, 78, 1024, kind="latent", cache_from_prev=True),
    3: Workload(3, "upsample_block", 2, 1, 512, 8, 88, 156, 512, kind="upsample"),
    4: Workload(4, "fullres_resblock", 3, 1, 256, 16, 352, 624, 256, kind="resblock",
                cache_from_prev=True, channel_offsets=True),
    5: Workload(5, "output_head", 4, 1, 256, 16, 352, 624, 12, kind="head"),
}


def conv_flops(n, t, h, w, k, c, taps=27):
    """Algorithmic FLOPs of one convolution: 2 * positions * K * C * taps (padded taps counted)."""
    return 2.0 * n * t * h * w * k * c * taps

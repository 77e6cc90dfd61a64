"""Seeded synthetic inputs, shared by the tests, the bench and the smoke check.

This module only draws numbers. It holds none of the arithmetic of GroupNorm,
SiLU or the convolutions, so both the CPU oracle and the GPU path can consume
its tensors without sharing any of the method's code.

Generator (counter-based, so any element can be drawn independently and the
same tensor comes out on the CPU or on a GPU):

* ``mix64`` is the SplitMix64 output function (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014): add the
  golden gamma 0x9E3779B97F4A7C15, then xor-shift 30 / multiply
  0xBF58476D1CE4E5B9 / xor-shift 27 / multiply 0x94D049BB133111EB /
  xor-shift 31, all modulo 2**64.
* The key of a tensor is ``mix64(seed * 2**16 + tensor_id)`` and element ``i``
  draws ``r = mix64(key + i)``.
* Normals: Box-Muller on two 24-bit uniforms cut from ``r``:
  ``u1 = (r >> 40 + 0.5) / 2**24`` (never 0), ``u2 = ((r >> 16) & 0xFFFFFF) / 2**24``,
  ``z = sqrt(-2 ln u1) * cos(2 pi u2)``, computed in float64, then scaled and
  rounded once to the requested dtype (round to nearest even).
* Uniforms on [lo, hi): ``lo + (hi - lo) * (r >> 11) / 2**53``.
"""
from __future__ import annotations

import math

import torch

_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _s64(v: int) -> int:
    """An unsigned 64-bit constant as the signed int64 torch stores."""
    v &= (1 << 64) - 1
    return v - (1 << 64) if v >= (1 << 63) else v


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 lanes (torch's >> is arithmetic)."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def mix64(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output of state ``z`` (int64 lanes, arithmetic mod 2**64)."""
    z = z + _s64(_GAMMA)
    z = (z ^ _srl(z, 30)) * _s64(_M1)
    z = (z ^ _srl(z, 27)) * _s64(_M2)
    return z ^ _srl(z, 31)


def mix64_int(z: int) -> int:
    """Pure-Python SplitMix64 on one word; the reference the tensor code is tested against."""
    m = (1 << 64) - 1
    z = (z + _GAMMA) & m
    z = ((z ^ (z >> 30)) * _M1) & m
    z = ((z ^ (z >> 27)) * _M2) & m
    return z ^ (z >> 31)


def _key(seed: int, tensor_id: int) -> int:
    k = mix64_int(((seed << 16) + tensor_id) & ((1 << 64) - 1))
    return _s64(k)


_CHUNK = 1 << 24


def _draw(seed: int, tensor_id: int, numel: int, device, fn, dtype) -> torch.Tensor:
    """``fn(words, index)`` over elements [0, numel), chunk by chunk, into a flat ``dtype`` tensor."""
    key = _key(seed, tensor_id)
    out = torch.empty(numel, dtype=dtype, device=device)
    for start in range(0, numel, _CHUNK):
        n = min(_CHUNK, numel - start)
        idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
        out[start:start + n] = fn(mix64(idx + key), idx).to(dtype)
    return out


def _normal_from_words(r: torch.Tensor) -> torch.Tensor:
    u1 = (_srl(r, 40).to(torch.float64) + 0.5) * 2.0 ** -24
    u2 = (_srl(r, 16) & 0xFFFFFF).to(torch.float64) * 2.0 ** -24
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def normal(shape, seed: int, tensor_id: int, std: float = 1.0, mean=0.0,
           dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """N(mean, std**2) of ``shape``, drawn in float64 and rounded once to ``dtype``.

    ``mean`` is a number or a 1-D tensor over the last dimension (a per-channel
    offset of a channels-last tensor); it is added in float64 before the rounding.
    """
    numel = math.prod(shape)
    if torch.is_tensor(mean):
        m = mean.to(device=device, dtype=torch.float64).reshape(-1)
        last = shape[-1]
        assert m.numel() == last

        def fn(r, idx):
            return _normal_from_words(r) * std + m[idx % last]
    else:
        def fn(r, idx):
            return _normal_from_words(r) * std + mean
    return _draw(seed, tensor_id, numel, device, fn, dtype).reshape(shape)


def uniform(shape, seed: int, tensor_id: int, lo: float, hi: float,
            dtype=torch.float32, device="cpu") -> torch.Tensor:
    """U[lo, hi) of ``shape`` with 53-bit resolution, rounded once to ``dtype``."""
    numel = math.prod(shape)
    return _draw(seed, tensor_id, numel, device,
                 lambda r, idx: lo + (hi - lo) * (_srl(r, 11).to(torch.float64) * 2.0 ** -53),
                 dtype).reshape(shape)


# Tensor ids within one configuration's seed.
X, GAMMA1, BETA1, W1, X_PREV, OFFSETS, GAMMA2, BETA2, W2, W_UP = range(10)
W_TIME, X_BLOCK = 10, 11          # the temporal x2's weight; an up block's input (its shortcut source)

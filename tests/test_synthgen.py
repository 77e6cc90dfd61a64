"""The seeded input generator (CPU): its counter-based words, the distributions it draws and
the property the samplers rely on -- any element, or any leading run of frames, can be
drawn alone and equals the same elements of the whole tensor."""
import math

import numpy as np
import torch

import synthgen as sg
from synthgen.workloads import WORKLOADS


def test_mix64_tensor_matches_scalar():
    idx = torch.tensor([0, 1, 2, 12345, 2 ** 40 + 7, -5, 2 ** 63 - 1], dtype=torch.int64)
    got = sg.mix64(idx)
    for i, v in zip(idx.tolist(), got.tolist()):
        want = sg.mix64_int(i & ((1 << 64) - 1))
        assert v & ((1 << 64) - 1) == want


def test_normal_moments_and_rounding():
    x = sg.normal((1 << 20,), 3, sg.X, std=2.0, mean=1.0, dtype=torch.float32).double()
    assert abs(x.mean().item() - 1.0) < 0.01
    assert abs(x.std().item() - 2.0) < 0.01
    b = sg.normal((4096,), 3, sg.X, std=2.0, mean=1.0)                 # bf16: one rounding of the same draw
    f = sg.normal((4096,), 3, sg.X, std=2.0, mean=1.0, dtype=torch.float64)
    assert torch.equal(b, f.to(torch.bfloat16))


def test_uniform_range():
    u = sg.uniform((1 << 16,), 1, sg.OFFSETS, -4.0, 4.0, dtype=torch.float64)
    assert u.min().item() >= -4.0 and u.max().item() < 4.0
    assert abs(u.mean().item()) < 0.05


def test_elements_drawn_alone_equal_the_whole():
    wl = WORKLOADS[4].scaled(t=5, h=6, w=7)
    whole = wl.x()
    assert torch.equal(wl.x(frames=2).view(torch.int16), whole[:, :2].view(torch.int16))
    # the per-channel offsets follow the channel index of every element
    off = wl.offsets().double()
    assert abs((whole.double().mean(dim=(0, 1, 2, 3)) - off).abs().max().item()) < 1.5
    assert math.prod(whole.shape) == wl.numel and np.isfinite(whole.float().numpy()).all()

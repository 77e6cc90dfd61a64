"""Pins of the oracle's bf16 decoding and single rounding (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import bf16


def test_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000, 0x0080], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, -0.0, 2.0 ** -126]
    got = bf16.decode(bits)
    assert got.tolist() == want
    assert np.signbit(got[4])


def test_round_matches_torch_on_fp32_values():
    # fp32 -> bf16 in torch is one RNE rounding; on fp32-representable inputs ours must agree.
    g = torch.Generator().manual_seed(0)
    v = torch.randn(200000, generator=g, dtype=torch.float32) * torch.exp(torch.randn(200000, generator=g) * 8)
    v = torch.cat([v, torch.tensor([0.0, -0.0, 1e-40, -3e-39, 6e-39, 3.3e38, -3.39e38])])
    want = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16.round_rne(v.numpy().astype(np.float64))
    assert np.array_equal(got, want)


def test_round_ties_to_even_and_single_rounding():
    cases = {
        1 + 2.0 ** -8: 0x3F80,               # tie between 1 and 1+2^-7 -> even (1.0)
        1 + 3 * 2.0 ** -8: 0x3F82,           # tie -> even significand (1 + 2^-6)
        1 + 2.0 ** -8 + 2.0 ** -40: 0x3F81,  # just above the tie: up. Via fp32 it would tie to 1.0
        -(1 + 2.0 ** -8 + 2.0 ** -40): 0xBF81,
        2.0 ** -134: 0x0000,                 # half the smallest subnormal: tie -> 0 (even)
        3 * 2.0 ** -134: 0x0002,             # 1.5 quanta -> 2 quanta
        2.0 ** -134 + 2.0 ** -160: 0x0001,   # above the tie: up to the smallest subnormal
        (2 - 2.0 ** -7) * 2.0 ** 127: 0x7F7F,
        (2 - 2.0 ** -8) * 2.0 ** 127: 0x7F80,  # tie at the top -> even -> infinity
        -(2 - 2.0 ** -7 + 2.0 ** -10) * 2.0 ** 127: 0xFF7F,  # below the top tie: max
        -(2 - 2.0 ** -9) * 2.0 ** 127: 0xFF80,              # above it: -infinity
    }
    got = bf16.round_rne(np.array(list(cases.keys())))
    assert [int(b) for b in got] == list(cases.values())


def test_round_decode_roundtrip_all_finite_bf16():
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    vals = bf16.decode(bits)
    finite = np.isfinite(vals)
    back = bf16.round_rne(vals[finite])
    assert np.array_equal(back, bits[finite])


@pytest.mark.parametrize("a,b,d", [(0x0000, 0x8000, 0), (0x3F80, 0x3F81, 1), (0x0001, 0x8001, 2),
                                   (0x3F80, 0xBF80, 2 * 0x3F80)])
def test_ulp_distance(a, b, d):
    assert int(bf16.ulp_distance(np.uint16(a), np.uint16(b))) == d

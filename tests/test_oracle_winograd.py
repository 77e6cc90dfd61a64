"""Pins of the oracle's Winograd F(4x4,3x3) form of the causal convolution (CPU only).

Against: the interpolation construction the three tables come from (rows of G and columns
of A^T are the monomials at the points 0, 1, -1, 2, -2 and infinity), the 1-D F(4,3)
identity (four outputs of a 3-tap correlation from six products), brute force of the
weight and input transforms, and the identity that matters -- the Winograd form equals the
direct causal convolution (oracle.conv) to fp64 rounding, borders and ragged tiles included.
"""
import numpy as np
import pytest

from oracle import conv as oconv
from oracle import winograd as ow

POINTS = [0.0, 1.0, -1.0, 2.0, -2.0]


def test_tables_follow_the_interpolation_points():
    # A^T column a = (1, p, p^2, p^3) for the finite points, (0, 0, 0, 1) for infinity
    for a, p in enumerate(POINTS):
        np.testing.assert_array_equal(ow.AT[:, a], [1.0, p, p * p, p ** 3])
    np.testing.assert_array_equal(ow.AT[:, 5], [0, 0, 0, 1])
    # G row a is proportional to (1, p, p^2) (the filter polynomial at p), infinity: (0, 0, 1)
    for a, p in enumerate(POINTS):
        row = ow.G[a]
        lead = row[0]
        assert lead != 0
        np.testing.assert_allclose(row / lead, [1.0, p, p * p], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(ow.G[5], [0, 0, 1])


def test_one_dimensional_f43_identity():
    """y_m = sum_r g_r d_{m+r} (m = 0..3) equals A^T [(G g) * (B^T d)] for random g, d."""
    rng = np.random.default_rng(3)
    for _ in range(50):
        g = rng.standard_normal(3)
        d = rng.standard_normal(6)
        direct = np.array([sum(g[r] * d[m + r] for r in range(3)) for m in range(4)])
        wino = ow.AT @ ((ow.G @ g) * (ow.BT @ d))
        np.testing.assert_allclose(wino, direct, rtol=1e-13, atol=1e-13)


def test_weight_transform_brute_force():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((3, 3, 3, 3, 5))
    u = ow.weight_transform(w)
    for a in range(6):
        for b in range(6):
            for k in range(3):
                for dt in range(3):
                    for c in range(5):
                        want = sum(ow.G[a, r] * ow.G[b, s] * w[k, dt, r, s, c] for r in range(3) for s in range(3))
                        assert abs(u[a, b, k, dt, c] - want) <= 1e-14


def test_input_transform_patches_brute_force():
    """V of the corner and the last (ragged) tiles from explicitly gathered, zero-padded patches."""
    rng = np.random.default_rng(5)
    p = rng.standard_normal((1, 2, 7, 10, 3))                 # tiles 2 x 3, the last ones ragged
    v = ow.input_transform(p)
    assert v.shape == (6, 6, 1, 2, 2, 3, 3)
    for (i, j) in [(0, 0), (1, 2), (0, 2), (1, 0)]:
        d = np.zeros((6, 6, 3))
        for r in range(6):
            for s in range(6):
                y, x = 4 * i - 1 + r, 4 * j - 1 + s
                if 0 <= y < 7 and 0 <= x < 10:
                    d[r, s] = p[0, 1, y, x]
        for c in range(3):
            np.testing.assert_allclose(v[:, :, 0, 1, i, j, c], ow.BT @ d[:, :, c] @ ow.BT.T, rtol=0, atol=1e-13)


@pytest.mark.parametrize("n,t,h,w,c,k,cache,bias,res", [
    (1, 3, 8, 8, 4, 3, True, False, False),     # whole tiles
    (2, 2, 7, 9, 5, 4, True, True, True),       # ragged tiles in both directions, two samples
    (1, 1, 5, 6, 3, 2, False, True, False),     # T = 1, zero cache
    (1, 4, 1, 1, 2, 2, True, False, False),     # a single pixel
    (1, 2, 4, 13, 3, 5, False, False, True),    # one tile row
])
def test_winograd_equals_direct_conv(n, t, h, w, c, k, cache, bias, res):
    rng = np.random.default_rng(n + t + h + w + c + k)
    a = rng.standard_normal((n, t, h, w, c))
    wt = rng.standard_normal((k, 3, 3, 3, c))
    ci = rng.standard_normal((n, 2, h, w, c)) if cache else None
    b = rng.standard_normal(k).astype(np.float32) if bias else None
    r = rng.standard_normal((n, t, h, w, k)) if res else None
    o1, c1 = oconv.causal_conv3d(a, wt, ci, b, r)
    o2, c2 = ow.causal_conv3d(a, wt, ci, b, r)
    assert np.array_equal(c1, c2)
    assert np.abs(o1 - o2).max() <= 1e-12 * np.abs(o1).max()


def test_winograd_causality():
    """Output frame t depends on frames <= t only, as the direct form."""
    rng = np.random.default_rng(6)
    a = rng.standard_normal((1, 4, 6, 9, 3))
    wt = rng.standard_normal((2, 3, 3, 3, 3))
    o, _ = ow.causal_conv3d(a, wt)
    b = a.copy()
    b[:, 2] += 1.0
    ob, _ = ow.causal_conv3d(b, wt)
    assert np.array_equal(o[:, :2], ob[:, :2])
    assert not np.allclose(o[:, 2:], ob[:, 2:])

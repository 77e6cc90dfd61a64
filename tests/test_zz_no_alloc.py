"""gn_silu_stats_noalloc (the statistics entry point that allocates nothing) through the C ABI,
against gn_silu_stats on the same inputs: two calls in a row, the second on a smaller input,
so that the shared scratch array's leftover contents from the first call cannot leak into the
second. With 32 groups both entry points use the same partial blocks: the results are
bitwise equal (and within 1e-12 of the oracle's statistics)."""
import ctypes

import numpy as np
import pytest
import torch

import silu_gn_amd as sga
import synthgen as sg
from oracle import groupnorm as ogn
from tests.helpers import vals

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _noalloc_raw(x, groups, stats):
    """The raw C call (no binding logic beyond pointers and the stream)."""
    lib = sga.load_library()
    n, t, h, w, c = x.shape
    rc = lib.gn_silu_stats_noalloc(ctypes.c_void_p(x.data_ptr()), sga.sgn_dims(n, t, h, w, c), groups,
                                   ctypes.c_void_p(stats.data_ptr()),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib.sgn_last_error().decode()


@pytest.mark.parametrize("shapes,groups", [
    (((2, 5, 33, 47, 256), (1, 2, 7, 9, 256)), 32),       # larger, then smaller (fewer blocks)
    (((1, 4, 44, 78, 1024), (1, 1, 3, 5, 64)), 32),       # the latent shape, then a tiny one
    (((1, 3, 16, 16, 2048), (1, 2, 4, 4, 2048)), 2048),   # one channel per group: fewer blocks
])
def test_noalloc_stats_matches_workspace_entry_point(shapes, groups):
    for i, shape in enumerate(shapes):
        print("case noalloc", i, shape, groups, flush=True)
        x = sg.normal(shape, 40 + i, sg.X, mean=0.3).to(DEV)
        ref = sga.gn_silu_stats(x, groups)
        got = torch.full_like(ref, float("nan"))
        _noalloc_raw(x, groups, got)
        torch.cuda.synchronize()
        r, g = ref.cpu().numpy(), got.cpu().numpy()
        if groups <= 128:
            assert np.array_equal(r, g)
        np.testing.assert_allclose(g, r, rtol=1e-12, atol=1e-14)
        mean, var = ogn.group_stats(vals(x), groups)
        np.testing.assert_allclose(g[..., 0], mean, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(g[..., 1], var, rtol=1e-12, atol=1e-14)


def test_noalloc_rejects_too_many_groups():
    lib = sga.load_library()
    x = torch.zeros((200, 1, 1, 1, 2048), dtype=torch.bfloat16, device=DEV)
    stats = torch.empty((200, 2048, 2), dtype=torch.float64, device=DEV)
    rc = lib.gn_silu_stats_noalloc(ctypes.c_void_p(x.data_ptr()), sga.sgn_dims(200, 1, 1, 1, 2048), 2048,
                                   ctypes.c_void_p(stats.data_ptr()), None)
    assert rc == -1 and b"scratch" in lib.sgn_last_error()

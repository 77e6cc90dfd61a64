"""CPU oracle for the silu(group_norm(x)) -> causal conv3d decoder path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The library in
``silu_gn_amd`` never calls it, and it shares no code with that library: it is
the plain definition of each operation, evaluated in float64 with numpy
(``numpy.matmul`` is the only library primitive used for the contractions).

What each module follows (pages: WanGP ``shared/kernels/group_norm_silu.py``;
FastVideo ``wan22_vae_decode/solution/binding.cpp``):

* ``bf16``       -- bf16 decoding and ONE round-to-nearest-even from float64
                    (group_norm_silu.py docstring: "one rounding to the output dtype").
* ``groupnorm``  -- per (sample, group) mean and biased variance; z = (x - mean)
                    / sqrt(var + eps) * gamma + beta; silu(z) = z / (1 + e^-z)
                    (group_norm_silu.py docstring and its apply kernel).
* ``rmsnorm``    -- the per-position RMS norm + SiLU the pages' decoder runs before its
                    output head (binding.cpp, the comment above Decoder::output_head):
                    z = x * gain / sqrt(mean_c(x^2) + eps), silu(z). The formula is
                    not printed on the pages; this is the usual RMS norm (the reading).
* ``conv``       -- the causal 3x3x3 convolution over cat(cache, input) with
                    1-pixel spatial zero padding and the 2-frame cache
                    (binding.cpp, Decoder::conv); nearest-x2 upsample + 3x3
                    convolution in its direct form and, only to check the
                    identity, the four 2x2 phases (binding.cpp, prepare());
                    the output head with a 2x2 depth-to-space.
* ``upblock``    -- the rest of an up block (binding.cpp, the seam after the resnets of
                    blocks 0 and 1, and the resampler's last pass): the causal 3x1x1 time
                    convolution writing two frames per input frame, the first pass's first
                    frame passed through; the DupUp3D shortcut (channel repeat, then
                    unfold to ft x fs x fs). Neither formula is printed on the pages; the
                    module docstring states the readings.

* ``winograd``   -- the causal 3x3x3 convolution through F(4x4,3x3) (binding.cpp,
                    prepare(): the 6x3 weight transform G, each of the 36 components
                    keeping the causal 3-tap temporal convolution; Decoder::conv: input
                    transform, per-component temporal products, output transform). The
                    input and output transforms are those of the same interpolation points
                    (the pages print G only); pinned by the identity with ``conv``.

Every function is pinned by ``tests/test_oracle_*.py`` against brute force,
closed forms, invariants or an independent library routine. Parity unpinned:
agreement with the real Wan2.2 decoder (trained weights, real latents, the
head's channel order), which needs data this repository does not have.
"""
from . import bf16, groupnorm, conv, rmsnorm, upblock, winograd  # noqa: F401

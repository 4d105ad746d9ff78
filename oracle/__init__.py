"""CPU reference (oracle) for MLA latent-cache decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything in this package; only
the tests, the smoke check and the benchmark's CPU-baseline leg use it.

The oracle is plain numpy in float64.  It computes MLA the non-absorbed way
(explicit per-head up-projection of K and V from the latent cache, then
ordinary softmax attention) and, separately, the absorbed form used to check
the intermediates of each library call.  It shares no code with the GPU path.
"""

from . import codecs, accounting, mla_ref  # noqa: F401

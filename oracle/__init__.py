"""CPU fp64 oracle for cross-layer shared-KV attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg call it.
It shares no code with the HIP library (no kernels, headers, helpers or
constant tables); both sides only consume the seeded tensors of ``datagen``.

The oracle computes the plain definitions, in float64, from logical
(unpaged) tensors:

* ``attention``  -- effective K/V of a layer through an explicit layer->source
                    map, single-query decode attention, causal / non-causal
                    prefill attention, and the factorized (basis + low-rank
                    int8 residual) key/value reconstruction.
* ``plan``       -- which layers own cached K/V, the owner-slot numbering and
                    the validity rules of a sharing map.
* ``factorize``  -- the factorized cache's write side: a layer pair's basis,
                    a layer's residual directions (leading singular vectors)
                    and the encoder (pair coefficients, int8 residual codes,
                    fp16 scale per token).
* ``router``     -- the token router's attention statistics (entropy, peak
                    probability of each decode query) and its rank choice.

Every function is pinned by the CPU tests to something other than itself
(closed forms, a library routine, invariants, brute force); none is marked
"parity unpinned".
"""
from . import attention, factorize, plan, router  # noqa: F401

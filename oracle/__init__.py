"""Plain float64 CPU oracle for compressed-domain KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, header, table or constant
generator with the HIP library; both sides only receive the same seeded
inputs from ``synth``.

The oracle follows three web pages, cited by title and section:

* "turbo4 post-mortem" -- the turboquant_plus article on reviving the turbo4
  KV-cache format (sections 1-10),
* "TurboQuant Triton deep dive" -- the article on the three tricks of the
  fused Triton decode kernels (sections "nine-step path", "trick 1",
  "trick 2", "trick 3", "how the kernels compose", "write path"),
* "PolarQuant-KV" -- the PolarQuant-KV consumer-GPU article (sections 1-6).

Modules
-------
codebook   scalar quantizer tables for N(0, 1/d) (quantile means, Lloyd-Max)
prng       splitmix64 stream, rotation signs, Box-Muller QJL matrix
rotation   Walsh-Hadamard + random-sign rotation
formats    encoders / block packers / decoders for PQ4, PQ3, TQ3K, GQ2V, GQ4V
attention  textbook softmax attention over dequantized caches, split/combine

Every function here is pinned by ``tests/test_oracle_*.py`` to something other
than itself (printed page values, textbook tables, closed forms, invariants,
brute force).  The only result without an external pin is the end-to-end
attention output on random caches ("parity unpinned" against the pages: no
worked example of bytes or outputs is printed); it rests on the pinned parts.
"""

from . import codebook, prng, rotation, formats, attention  # noqa: F401

"""fp64 CPU oracle for ResidualQuant decode attention over a packed, paged KV cache.

TEST INFRASTRUCTURE ONLY. This package exists to check the HIP library. Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The product path (the HIP library under
``looped_transformer_decode_rq_amd/`` and its Python binding) never imports,
links or calls it, and the two share no code, header, table or helper; the only
common dependency is the seeded input generator in ``workloads/``, which holds
none of the method's arithmetic.

Every function is a plain, slow, step-by-step statement of what the method
computes, in float64, following the pages' order:

* ResidualQuant: KV Cache Quantization for Looped Transformers with 2-Bit
  Residuals (arXiv 2610.10381, listing page with the English abstract) --
  final-loop reference, low-precision residuals of the other loops,
  least-squares scaling, rotations on the residuals, loop-wise mixed precision.
* rit.work summary of the same paper, section "how the KV cache of each pass
  is restored" -- reference = last pass; per-difference scale by least squares;
  channel-space rotation calibrated per (layer, head, K|V) and shared by all
  tokens and passes; INT4 reference, INT2 differences with tunable step and
  offset; the current token's intermediate KV kept in BF16 until the final
  pass; reconstruction inside attention.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
closed forms, invariants, a hand-derived worked example (``tests/golden/``) and
library routines -- never against the HIP path.
"""
from .rq_oracle import *  # noqa: F401,F403
from .rq_oracle import __all__  # noqa: F401

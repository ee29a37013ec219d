"""TEST INFRASTRUCTURE: fp64 CPU oracle for the chunked gated delta rule.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never imports it and shares no code with it.

``gdn_fwd`` / ``gdn_bwd`` wrap the plain C token loop in ``gdn_oracle.c``
(built with gcc, no fast-math, no BLAS).  ``shortconv_fwd`` /
``shortconv_bwd`` are the short causal convolution with its boundary state.
``plan`` holds a plain search for the hybrid-cost chunk boundaries.  Method source: "Pith review of StateFlow:
Sequence Pipeline Parallelism for Long-Context Modeling with Linear
Recurrence", "What carries the argument" (Eqs. 5 and 7, cost model Eq. 9) and
"Referee Report" major comment 1 (gated delta rule, Eq. (1)).
"""
from .gdn import gdn_fwd, gdn_bwd, gdn_fwd_chained, gdn_bwd_chained, build, lib_path  # noqa: F401
from .gdn import shortconv_fwd, shortconv_bwd  # noqa: F401

"""FP64 CPU oracle for the IsoQuant packed-KV path.

TEST INFRASTRUCTURE ONLY. Nothing in the product (the HIP library and its
Python binding) imports, calls, links or executes anything in this package.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.

The oracle shares no code, table or constant generator with the HIP path.  It
is written from the pages of:

* "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
  Compressed-Space Attention" (arXiv 2608.08081), §3.2 Algorithm 1 and
  eq. (2), §3.3, §3.4 Table 2, Appendices A and B;
* "IsoQuant: Hardware-Aligned SO(4) Isoclinic Rotations for LLM KV Cache
  Compression" (arXiv 2603.28430), abstract (Full / Fast variants).

Every function in :mod:`oracle.isoquant` is pinned by a ``-m "not gpu"`` test
to something other than itself (closed forms, textbook values, invariants,
brute force).  The packed-code values themselves have no worked example on the
pages: against the pages, code parity is unpinned beyond those closed forms.
"""

from .isoquant import *  # noqa: F401,F403

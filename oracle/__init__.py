"""CSA2 oracle: a plain, slow, float64 CPU statement of the CSA2 hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product (the HIP
library and its Python binding) never imports it and shares no code with it.

Modules:
* ``formats``   — bfloat16 / E4M3 / E2M1 tables and the FP4 block codec.
* ``csa2``      — compress, RoPE, store, indexer score, top-k, HSI pool,
                  sparse attention with window, Full/Reindex/Reuse group.
* ``footprint`` — bytes-per-token arithmetic from the codec's byte counts.

Parity pins: every function is pinned by a CPU test against something other
than itself (enumerated tables, library conversions, brute force, closed
forms, invariants), except two formulas the pages do not print, which are
"parity unpinned" for their form (their invariants are still tested): the
indexer score, and the YaRN rotary interpolation and temperature
(``csa2.rope_freqs``, ``csa2.logit_temperature``), of which the pages give
only the original length and the factor.
"""
from . import csa2, footprint, formats  # noqa: F401

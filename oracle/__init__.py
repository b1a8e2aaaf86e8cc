"""Plain, slow CPU oracle of the CSA2 hot path (NumPy, fp64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import anything from this package.  It
shares no code with the HIP library or its Python binding, and imports neither.

Every function follows the definition of what the method computes, with no
blocking, fusion or reordering beyond it:

* ``formats``  - E4M3 / E2M1 / E8M0 / bf16 decoding from the bit definitions.
* ``write_side`` - encoding new pool entries (MXFP4 latent, E4M3 keys) and
                 window rows into their ring.
* ``csa2``     - indexer score, Top-K with the lower-index tie-break, the
                 hierarchical candidate pool, the Full / Reindex / Reuse mode
                 schedule, attention over the union of the selected FP4 global
                 entries and the FP8 window, and causal chunked prefill.

Parity is pinned (tests/test_oracle_*.py) by closed forms, exhaustive code
enumeration, brute force on tiny inputs, library routines (torch CPU casts and
scaled_dot_product_attention) and invariants.  The functions whose *formula*
is a reading of silent pages (the indexer score form, the index-key shape, one
pool for all layers, per-layer inputs, the causal rule and the planting recipe)
are pinned only for self-consistency: parity unpinned for those readings.
"""
from . import formats, csa2, write_side  # noqa: F401

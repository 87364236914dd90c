"""Plain CPU oracle for tree verification (test infrastructure only).

This package is the checker, not the product: only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it.  It is written in
NumPy float64 from the pages' definitions, step by step, with no blocking,
fusion or reordering, and shares no code with the HIP library.

Modules and the passage each follows:

* ``mask``  ancestor-or-self mask, depths and position ids of a flattened
  draft tree (serve-integration spec, "2. Verify: tree attention mask" and
  "Layout contract"; DDTree validation post, "The Successful Test").
* ``attn``  tree-masked attention over the paged context plus the ancestor
  nodes, with an optional sliding window (serve-integration spec, "2. Verify").
* ``walk``  greedy tree walk with the bonus token (serve-integration spec,
  "What's proven" and "3. Rejection sampler: tree walk").
* ``gdn``   Gated DeltaNet outputs along each node's root path, with no state
  written back (DFlash-TfM summary, "3. Rollback-vrije Boom-verificatie voor
  GDN"); also the masked triangular-solve form of the same computation.
* ``kvcommit``  the accepted path's keys and values written into the paged
  cache at positions ctx_len + s (serve-integration spec, layout contract).
* ``treebuild``  draft-tree construction: per-depth top-k of the draft
  distribution and best-first growth on cumulative log-probability (DDTree
  validation post, "The Failed First Attempt"; DFlash-TfM summary,
  "2. Boomconstructie").

Every function is pinned by tests under ``tests/`` that check it against
values printed on the pages, closed forms, invariants, brute force on tiny
inputs or library routines.
"""
from . import attn, gdn, kvcommit, mask, treebuild, walk  # noqa: F401

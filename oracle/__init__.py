"""CPU oracle for exact attention: test infrastructure, never part of the product path.

Only the tests, the smoke entry point and the bench's CPU-baseline leg may
import anything under this package.  It shares no code, constants or helpers
with the HIP library and it imports nothing from the product package.

Modules:

* ``attention`` -- the plain definition of causal/unmasked scaled-dot-product
  attention (forward O and log-sum-exp L) and its analytic gradient, in
  float64 with the score matrix materialised.
* ``online`` -- the online normaliser (m, l) recurrence, its associative merge,
  a block-wise forward in the loop order of the pages, and the "broken"
  variant without the rescale (a negative control).
* ``traffic`` -- count-only walks of the pages' one-head lesson kernels and
  their closed forms for global traffic, multiply-adds, exponentials, barriers
  and shared-memory traffic, plus the algorithmic work of the attention hot
  path used for measurement.

Every function is pinned by tests under ``tests/`` (``-m "not gpu"``).
"""

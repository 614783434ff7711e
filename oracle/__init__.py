"""Oracle for the gated-delta-rule chunked-prefill forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import, call, link or execute anything in this package.  The product
path (the HIP library and its Python binding) never touches it, and this
package imports nothing from the product path.

Two independent CPU implementations, both in fp64:

* ``recurrent``  -- the token-by-token recurrence (plain C, threaded), the
  definition the chunkwise method must reproduce;
* ``chunkwise``  -- a literal numpy evaluation of the chunkwise formulas
  (local gate cumsum, gated beta*K K^T, exact unit-lower inverse, WY factors,
  the serial chunk-state recurrence, the output), including the
  context-parallel pre-process and fix-up.  It exposes the intermediates.

How each function is pinned to something other than itself is listed in the
test files ``tests/test_oracle_*.py``.
"""

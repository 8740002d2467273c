"""fp64 CPU oracle for the ring-attention hot path -- TEST INFRASTRUCTURE.

Only the test-suite (``tests/``), the smoke check (``__graft_entry__.smoke``)
and the CPU-baseline leg of ``bench.py`` may import anything from here.  The
product path (``long_context_transformers_amd``) never imports it, and this
package imports nothing from the product.  The one module both sides share is
``ra_synth`` (seeded input draws, no attention arithmetic).

Modules:
  ``cref``   -- ctypes binding of ``ra_oracle.c`` (C99 + OpenMP, fp64):
                the plain definition of attention with an explicit mask,
                row-sampled, plus its closed-form gradient.
  ``npref``  -- NumPy fp64 forms: the dense definition, the pages' blocked
                ring procedure (both accumulator forms), the LogSumExp merge,
                and a pure-Python brute force for tiny inputs.
  ``build``  -- compiles ``ra_oracle.c`` into ``liboracle.so``.

Parity status of each function is listed in the module docstrings; every
function here is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_pins.py``.
"""

"""CPU oracle for absorbed MLA decode — TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The HIP path never
does, and this package imports nothing from the HIP path: the two share no
code.  Inputs come from ``deepseek_mla_latent_amd.inputs`` (random draws
only), passed in by the caller as numpy arrays.

Modules:

* ``mla_decode`` — fp64 numpy reference of the decode path, written the
  non-absorbed way (K and V up-projected per head), plus the plain
  definitions of the three library calls.
* ``mla_prefill`` — fp64 reference of prefill in multi-head form (order 1): K/V
  up-projection of every cached token, then per-head attention over them.
* ``mla_prepare`` — fp64 reference of the step before the path: the fused a-projection (a plain
  matmul), rotary position embedding, and the AppendKV scatter into the paged cache.
* ``fp8`` — E4M3 rounding and coding, block quantisation (128 x 128 weight blocks, 128-element
  activation vectors) and the two per-head products in FP8.
* ``flops`` — the pages' FLOP convention and the three computation orders of
  both absorptions, counted step by step from index extents; byte counts.

Every function is pinned by ``tests/test_oracle.py``, ``tests/test_oracle_prefill.py``,
``tests/test_oracle_prepare.py``, ``tests/test_oracle_fp8.py`` and ``tests/test_flops.py``
against what the pages print and against closed forms, special cases and
library routines (see each test's docstring).
"""

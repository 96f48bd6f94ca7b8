"""Plain, slow fp64 CPU oracle for the CSA2 global-attention path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: it is used by ``tests/``, by the
``smoke()`` check in ``__graft_entry__`` and by the ``cpu_baseline`` leg of
``bench.py``, and nowhere else.  It shares no code, table or constant
generator with the HIP library; the only thing the two sides have in common
is the seeded input generator (``long_context_sparse_csa2_amd.synth``), which
holds none of the method's arithmetic.

Sources (page titles as cited throughout):
  * "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
    (report digest) -- sections 2.3, 2.3.1, 2.3.2 and 2.4.4.
  * mer.dev commentary on DeepSeek-V4.1-Flash -- sections 2, 4.1-4.4 and 5.
  * paperglide summary of DeepSeek-V4 -- CSA and HCA walk-throughs (used only
    for the worked pooling example).
  * OCP Microscaling Formats (MX) v1.0 and OCP 8-bit Floating Point
    specifications for the bit-level E2M1 / E4M3FN / E8M0 definitions, which
    the pages name but do not spell out.

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` (spec code tables, printed constants, closed forms,
invariants, brute force on tiny inputs).  No function is "parity unpinned".
"""

from . import formats, csa2_ref  # noqa: F401

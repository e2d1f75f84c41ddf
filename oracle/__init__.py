"""fp64 CPU oracle for paged / block-sparse attention -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  The product path (``paged_kv_block_amd``) never
imports, links or runs anything in here, and nothing here imports the product.

Contents
--------
attention   plain fp64 NumPy definition of the attention result for the four
            entry points (block-sparse, paged prefill, paged decode, Sage).
bruteforce  a second, loop-only implementation for tiny inputs (math.fsum).
fp8         OCP E4M3FN decode written from the format's definition.
metadata    host-side metadata rules (validation status and first bad index)
            and the split/worklist policies, restated from the written spec.

Parity status
-------------
Every function here is pinned by ``tests/test_oracle_*.py`` (brute force, a
library SDPA routine, closed forms and the invariants the pages fix), except the
in-kernel fp8 quantisation of the Sage probabilities, which the pages do not
specify: the Sage oracle works on the *dequantized* inputs and the GPU result is
held to a tolerance only ("parity unpinned" for that design choice).
"""

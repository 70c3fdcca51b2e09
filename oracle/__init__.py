"""CPU oracle of one tensor-parallel rank's share of a Megatron-style sublayer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or runs
this package: only the test suite, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP path; the only thing the
two have in common is the seeded input generator module, which holds none of
the method's arithmetic.

Everything is computed in float64 NumPy from the exact values of the (bf16 or
fp32) inputs.  ``tp_oracle`` is the sublayer itself, ``analytic`` the closed
forms the pages print (pipeline bubble, all-reduce volumes, per-device
weights, GQA divisibility).

Parity status: every function here is pinned by tests under tests/ (identity
of the sharded and unsharded sublayer, brute force on tiny shapes, activation
closed forms and library routines, attention special cases, the pages'
printed values).  The GPU's bf16 rounding of H(t) and y(t) has no printed
value on the pages to pin against: it is judged against this oracle within
the stated tolerance only.
"""
from . import analytic, tp_oracle  # noqa: F401

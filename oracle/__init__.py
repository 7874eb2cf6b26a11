"""Oracle for the FlashBlock step and the LoSA-style sparse path.

TEST INFRASTRUCTURE ONLY.  A plain, slow, fp64 CPU implementation written from the
pages, sharing no code with the HIP library (cached_kv_prefix_amd).  Only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may import it; the library
never does.

Every function is pinned by -m "not gpu" tests to closed forms, brute force, a library
cross-check or invariants (tests/test_oracle_*.py).  No function is parity-unpinned.
"""
from . import attention, flashblock, losa  # noqa: F401

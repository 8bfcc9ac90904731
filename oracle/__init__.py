"""fp64 CPU oracles for the KDA forward operator.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg may import anything from here. The HIP product
path shares no code with it and never imports it.

* ``recurrent``  oracle-R: the token-by-token recurrence (C, fp64, OpenMP).
* ``chunkwise``  oracle-C: the chunkwise WY/UT form in numpy fp64, for small
  inputs and for intermediate values (g, A, T^{-1}, W, U, per-chunk states).
* ``epilogue``   the output epilogue: head-wise RMSNorm times a sigmoid gate.

Every function here is pinned by tests/test_oracle_pins.py against closed
forms, hand-worked examples and special cases named on the pages.
"""
from . import chunkwise, epilogue, recurrent  # noqa: F401

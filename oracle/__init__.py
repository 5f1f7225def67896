"""Plain fp64 CPU oracle for the Wan2.2 DiT self-attention step.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it. It
shares no code, constants or helpers with the HIP library; the only thing both
sides see is the seeded input data, which is generated elsewhere and handed in
as arrays.

What it computes (sources are the five web pages on Wan2.2 that define the
method; cited by page title and section):

* ``numerics``  -- round-to-nearest-even emulators for bfloat16 and OCP e4m3
  written from the format definitions.
* ``wan_ref``   -- full-width Q/K RMSNorm, the bf16 rounding point, 3-D RoPE
  over the (frame, row, column) latent grid, bidirectional softmax attention
  over the packed ``[Q|K|V]`` buffer, the per-tensor e4m3 quantisation, the
  chunked attention with log-sum-exp and the merge of two chunks.
* ``brute``     -- pure-Python loop versions of the same definitions for tiny
  inputs, used as one of the pins.

Parity status: every function here is pinned by closed forms, invariants,
library routines or brute force in ``tests/test_oracle_*.py``; the one thing
that is *parity unpinned* is agreement with a trained Wan2.2 checkpoint's RoPE
pairing convention (interleaved pairs are our reading), since no checkpoint or
golden tensor exists on the pages.
"""

from . import numerics, wan_ref, brute  # noqa: F401

"""CPU oracle of the sparse GQA global-attention path (test infrastructure).

This package is the plain, slow, float64 definition of what the GPU path
computes, written from the pages on Step-5-Preview's sparse GQA layers
("Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache", and the
Step 5 Preview architecture-blog summary).  It exists to check the HIP
library; it is NOT a fallback and is not on any product path.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library.

Modules
-------
``numerics``  bf16 / E4M3 rounding, written with integer bit operations and
              exact binary scaling.
``sgqa``      the four steps: proxy-key LayerNorm + RoPE and block merging,
              indexer query RMSNorm + RoPE and weighted-ReLU scores, causal
              top-k block selection, sparse GQA attention over the selected
              original K/V.

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: library casts and norms, closed-form invariants the pages state,
brute force on tiny inputs, dense causal attention as the all-blocks special
case, and the counts the pages print.  Two choices no page fixes -- the RoPE
pairing / frequencies and the LayerNorm-before-merge order -- are readings
and are marked "parity unpinned" where they are made.
"""
from . import numerics, sgqa  # noqa: F401

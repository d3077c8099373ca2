"""Independent fp64 CPU oracle for block-sparse video attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code, table or helper with the HIP library; both sides get their
inputs from the seeded generator in ``synth``.

Every function states what it computes and which passage of the source pages
it follows; where the pages leave a rule open, the reading taken is stated in
the function's docstring.

Parity status of each part (what pins it, see ``tests/test_oracle_*.py``):
  layout / permute ............ pinned (hand-enumerated grids, bijectivity)
  window / skiparse masks ..... pinned (closed-form counts, brute force)
  pooling / scores / top-k .... pinned (brute force, argsort cross-check)
  top-p with floor ............ pinned (prefix-mass properties, brute force)
  e4m3 codec / quantiser ...... pinned (format definition, torch casts)
  attention ................... pinned (brute-force dense, torch SDPA, closed forms)
  attention gradients ......... pinned (finite differences, torch autograd, closed forms)
  fp8 attention ............... parity unpinned beyond the tolerance gate
"""
from .layout import Layout
from . import layout, masks, routing, fp8, attention, attention_grad

__all__ = ["Layout", "layout", "masks", "routing", "fp8", "attention", "attention_grad"]

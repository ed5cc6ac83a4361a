"""CPU oracle for the ARK-ASR-3B int8 decoder step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything under this package: only tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP path.

Parity status per function (see each docstring for the passage it follows):
  every function here is pinned by tests under tests/ that check it against
  closed forms, brute force on tiny inputs, invariants fixed by the pages, or
  the pages' printed numbers.  The behaviour of the trained model (its
  transcripts, the verification table missing from the model card) is parity
  unpinned: no trained weights exist in this environment.  Two readings of
  the 3B adapter are parity unpinned as choices (the functions themselves
  are pinned): the GELU between its layers and its 4096 inner width (the
  pages print neither; the 0.6B parameter count pins the two-layer
  structure and an inner width of twice the hidden width there).  The
  audio encoder's structure is pinned by its printed parameter count; its
  readings of what the count cannot see are parity unpinned as choices:
  20 heads, rotary embedding (theta 10000) on q and k in every layer in
  addition to the positional table, int8 convolutions, LayerNorm eps 1e-5.
"""
from .ark import *  # noqa: F401,F403
from .ark import __all__  # noqa: F401

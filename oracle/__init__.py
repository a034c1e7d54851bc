"""CPU oracle for draft-guided mixed-precision block-sparse attention (DraftAttention2).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this package:
only the tests, the package's smoke check and the benchmark's CPU-baseline leg use it.  It shares
no code with the HIP library (no kernels, headers, helpers, tables or constant generators).

It is a plain, slow, step-by-step numpy implementation in fp64 of what the method computes, as
described in "DraftAttention2: Fast Video Diffusion with Low-Resolution-Guided Mixed-Precision
Attention" (newx.sg paper card: Abstract and AI Summary; pchao.org blog: section 方法概览 and the
Figure 2 and Figure 3 captions) and, for the reorder/restore framing, in "DraftAttention: Fast Video
Diffusion via Low-Resolution Attention Guidance" (pith.science, Abstract).  Quantisers emulate the
device grids exactly in IEEE fp32 (numpy float32 arithmetic is correctly rounded).

Modules, in pipeline order:
  layout     region geometry, pack (reorder + pad) and unpack (restore)
  draft      avg/max pooling, draft attention maps, lambda mix, per-head ranking and quota assignment
  quant      bf16 / e4m3fn / e2m1 rounding, per-block INT8, per-32-channel MXFP4, per-channel FP8 V
  attention  phased online-softmax attention over the 4-level block map
  pipeline   one layer end to end, per head
  dense      exact dense softmax attention (what the sparse operator approximates)

Every function states the passage it follows.  Where the pages leave a step open, the reading used
is stated in that function's module docstring as a numbered reading (R1..R30).

Parity status: every function is pinned by CPU tests (tests/test_oracle_*.py) against closed forms,
library routines, exhaustive brute force or invariants.  The end-to-end numbers are "parity unpinned"
against the pages: the pages print no worked example.
"""
from . import layout, quant, draft, attention, pipeline, dense  # noqa: F401
from .pipeline import run, run_head, HeadResult  # noqa: F401

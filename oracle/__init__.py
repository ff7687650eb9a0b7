"""Float64 CPU oracle for one context-parallel rank's share of causal ring attention.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
HIP path is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import it.  The product path
(``ring_attention_rank_amd``) never imports it, and the two share no code: no
kernels, helpers, tables or pre/post-processing.  The only thing both sides use
is the seeded input generator in ``synth/``, which holds none of the method's
arithmetic.

Sources (the three web pages it follows):

* "Context Parallelism (CP)" concept page (research-hub), section
  "Key math / How it works": ring of GPUs, blockwise attention with the online
  softmax, causal-mask imbalance and striped balancing.
* "primitive-context-parallel" skill page (curry-train), sections
  "What it does" and "Memory": contiguous ranges per rank, the one-other-rank
  KV buffer.
* Zero to Frontier, "distributed/context-expert" section, subsections
  "Splitting the sequence, and the one layer that objects" (ring steps, the
  running max / exp-sum / weighted value sum), "What context parallelism
  communicates" (bytes per KV block), "When the ring hides its communication"
  (4 n^2 d FLOPs per visible block), "The causal mask unbalances the sequence"
  (contiguous / zigzag / striped work) and "Ulysses, splitting by heads
  instead" (the all-to-all byte model and its break-even).

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` against something other than itself (brute force,
a library routine, closed forms, invariants, or figures printed on the pages).
"""

from .ring import (  # noqa: F401
    LAYOUTS,
    positions,
    ring_sources,
    init_state,
    block_partial,
    fold,
    ring_step_ref,
    finalize,
    ring_forward_ref,
    brute_attention,
    default_scale,
    doc_ids,
)
from .backward import (  # noqa: F401
    backward_prep_ref,
    block_backward_ref,
    ring_backward_ref,
)
from .counts import (  # noqa: F401
    chunk_assignment,
    causal_work,
    visible_pairs,
    tile_work,
    half_blocks_from_tiles,
    kv_block_bytes,
    cp_comm_bytes,
    ulysses_breakeven,
    overlap_min_tokens,
    visible_flops,
)

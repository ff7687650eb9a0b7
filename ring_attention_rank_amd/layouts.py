"""Where a rank's tokens sit in the global sequence (host-side set-up).

Zero to Frontier, "distributed/context-expert", section "The causal mask
unbalances the sequence", and the curry-train "primitive-context-parallel"
page, section "What it does":

* contiguous: rank r holds the r-th of n_cp equal runs (half-open range);
* zigzag: the sequence is cut into 2*n_cp chunks and rank r holds chunk r and
  its mirror 2*n_cp-1-r, in that order;
* striped: tokens are dealt round-robin, token t to rank t mod n_cp.

The ring passes blocks to the right, so at step b rank r holds the block that
started on rank (r - b) mod n_cp.
"""

import numpy as np


def rank_positions(T, n_cp, r, layout):
    """int32 global positions of rank r's tokens, in local order."""
    if not 0 <= r < n_cp:
        raise ValueError("rank out of range")
    if layout == "contiguous":
        if T % n_cp:
            raise ValueError("T must be a multiple of n_cp")
        n = T // n_cp
        return (r * n + np.arange(n)).astype(np.int32)
    if layout == "zigzag":
        if T % (2 * n_cp):
            raise ValueError("T must be a multiple of 2*n_cp")
        c = T // (2 * n_cp)
        idx = np.arange(c)
        return np.concatenate([r * c + idx, (2 * n_cp - 1 - r) * c + idx]).astype(np.int32)
    if layout == "striped":
        if T % n_cp:
            raise ValueError("T must be a multiple of n_cp")
        return (np.arange(T // n_cp) * n_cp + r).astype(np.int32)
    raise ValueError(f"unknown layout {layout!r}")


def ring_block_owner(n_cp, r, step):
    """Rank whose block rank r holds at ring step ``step``."""
    return (r - step) % n_cp


def document_start_of(pos, doc_starts):
    """int32 first global position of the document holding each position.

    Packed sequences (Zero to Frontier, "Splitting the sequence, and the one
    layer that objects": gathered keys and values make document masks easy):
    ``doc_starts`` are the increasing first positions of the documents, the
    first one 0.  A key is visible to a query under the document mask exactly
    when its position lies between the query's document start and the query
    itself, which is the lower bound the all-gather entry point takes.
    """
    starts = np.asarray(doc_starts, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    if starts.size == 0 or starts[0] != 0 or np.any(np.diff(starts) <= 0):
        raise ValueError("doc_starts must increase from 0")
    return starts[np.searchsorted(starts, pos, side="right") - 1].astype(np.int32)

"""Work, tile and byte counts of context-parallel attention, done properly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Zero to Frontier "distributed/context-expert" section prints exercise
stubs (``chunk_assignment``, ``causal_work``, ``cp_comm_bytes``,
``ulysses_breakeven``) whose bodies are placeholders.  Only their names and
arguments are kept; the bodies below follow the section's prose:

* "The causal mask unbalances the sequence": GPU i of a contiguous split
  computes i+1 blocks, the diagonal one half visible, so the last GPU does
  2*n_cp-1 times the first's work; zigzag (chunks i and 2*n_cp-1-i) and
  striped (round-robin) equalise it.
* "What context parallelism communicates": one GPU's keys and values are
  2*n*d_kv numbers, 4*n*d_kv bytes in 16 bits; the ring and the all-gather
  each deliver the other n_cp-1 blocks.
* "When the ring hides its communication": a fully visible n-by-n block costs
  4*n^2*d FLOPs over all heads (2 n^2 d for Q K^T, 2 n^2 d for the weighted
  values); the send hides when that compute outlasts shipping 4*n*d_kv bytes.
* "Ulysses, splitting by heads instead": an all-to-all keeps 1/n_cp of each
  GPU's buffer (Q and output of width d, K and V of width d_kv) and sends the
  rest; Ulysses wins once the group exceeds 1 + h/n_kv GPUs.
"""

from fractions import Fraction

import numpy as np


def chunk_assignment(n_gpus, layout, n_chunks=None):
    """Chunk ids held by each GPU, as a list per GPU.

    contiguous: n_gpus chunks, GPU i holds [i].
    zigzag: 2*n_gpus chunks, GPU i holds [i, 2*n_gpus-1-i].
    striped: single-token chunks dealt round-robin; ``n_chunks`` (the token
    count) is required.
    """
    if layout == "contiguous":
        return [[i] for i in range(n_gpus)]
    if layout == "zigzag":
        return [[i, 2 * n_gpus - 1 - i] for i in range(n_gpus)]
    if layout == "striped":
        if n_chunks is None:
            raise ValueError("striped needs the token count")
        return [list(range(i, n_chunks, n_gpus)) for i in range(n_gpus)]
    raise ValueError(f"unknown layout {layout!r}")


def causal_work(assignment):
    """Causal attention work of each GPU in chunk-pair blocks.

    A GPU's query chunk a needs key chunks b <= a of the whole sequence;
    b < a is a full block (1), b == a the diagonal block, counted as half
    visible (0.5).  The sequence's chunk count is the total over all GPUs.
    """
    total_chunks = sum(len(ch) for ch in assignment)
    out = []
    for chunks in assignment:
        w = Fraction(0)
        for a in chunks:
            if not (0 <= a < total_chunks):
                raise ValueError("chunk id out of range")
            w += a  # key chunks 0..a-1 are fully visible
            w += Fraction(1, 2)  # the diagonal chunk
        out.append(float(w))
    return out


def visible_pairs(q_pos, k_pos, causal=True):
    """Number of (query, key) pairs with k_pos <= q_pos (all pairs if not causal)."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    if not causal:
        return int(q_pos.size) * int(k_pos.size)
    ks = np.sort(k_pos)
    # searchsorted(right) = number of keys <= each query position
    return int(np.searchsorted(ks, q_pos, side="right").sum())


def tile_work(q_pos, k_pos, BM, BN, causal=True, q_doc=None, k_doc=None):
    """Classify every (query tile, key tile) pair of one block and count them.

    Tiles are consecutive runs of BM query rows and BN key rows (the last of
    each may be short).  A tile pair is *full* if every (query, key) pair in it
    is visible, *skipped* if none is, and *masked* otherwise.  Returns
    (full, masked, skipped).  The classes do not depend on the head.

    Computed by counting the visible pairs of every tile (query rows in
    slices so the visibility matrix stays small) and comparing the count with
    the tile's size.  With document ids (``q_doc``, ``k_doc``) a visible pair
    must also share its document.
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    n_q, n_k = q_pos.size, k_pos.size
    if n_q == 0 or n_k == 0:
        return 0, 0, 0
    n_qt, n_kt = -(-n_q // BM), -(-n_k // BN)
    docs = q_doc is not None
    if docs:
        q_doc = np.asarray(q_doc, dtype=np.int64)
        k_doc = np.asarray(k_doc, dtype=np.int64)
    if not causal and not docs:
        return n_qt * n_kt, 0, 0
    col_starts = np.arange(0, n_k, BN)
    col_sizes = np.minimum(col_starts + BN, n_k) - col_starts
    full = masked = skipped = 0
    rows_per_slice = max(BM, (1 << 22) // max(1, n_k) // BM * BM)
    for r0 in range(0, n_q, rows_per_slice):
        qp = q_pos[r0:r0 + rows_per_slice]
        vis = np.ones((qp.size, n_k), dtype=bool)
        if causal:
            vis &= k_pos[None, :] <= qp[:, None]
        if docs:
            vis &= k_doc[None, :] == q_doc[r0:r0 + rows_per_slice, None]
        vis = vis.astype(np.int32)
        per_col_tile = np.add.reduceat(vis, col_starts, axis=1)  # [rows][n_kt]
        row_starts = np.arange(0, qp.size, BM)
        counts = np.add.reduceat(per_col_tile, row_starts, axis=0)  # [tiles][n_kt]
        row_sizes = np.minimum(row_starts + BM, qp.size) - row_starts
        sizes = row_sizes[:, None] * col_sizes[None, :]
        full += int((counts == sizes).sum())
        skipped += int((counts == 0).sum())
        masked += int(((counts > 0) & (counts < sizes)).sum())
    return full, masked, skipped


def half_blocks_from_tiles(full, masked, chunk, BM, BN):
    """Causal work in half chunk-pair blocks from tile counts.

    When tiles nest inside chunks, a full chunk pair holds (chunk/BM)(chunk/BN)
    full tiles (2 half-blocks) and a diagonal chunk pair holds full tiles below
    its diagonal plus masked tiles on it, which add up to one half-block as
    2*full + masked.  Returned as an exact Fraction.
    """
    return Fraction(2 * full + masked, (chunk // BM) * (chunk // BN))


def kv_block_bytes(n, d_kv, bytes_per_elem=2):
    """Bytes of one GPU's key and value block: 2*n*d_kv numbers."""
    return 2 * n * d_kv * bytes_per_elem


def cp_comm_bytes(T, d, d_kv, n_cp, method, bytes_per_elem=2):
    """Bytes one GPU receives per attention layer in the forward pass.

    ring / allgather: the other n_cp-1 blocks of 2*n*d_kv numbers.
    ulysses: each GPU's buffer of n tokens (Q and output of width d, K and V
    of width d_kv) keeps 1/n_cp and sends the rest, so
    2*n*(d + d_kv)*bytes*(n_cp-1)/n_cp bytes cross the all-to-alls.
    """
    if T % n_cp:
        raise ValueError("T must be divisible by n_cp")
    n = T // n_cp
    if method in ("ring", "allgather"):
        return (n_cp - 1) * kv_block_bytes(n, d_kv, bytes_per_elem)
    if method == "ulysses":
        b = Fraction(n * (2 * d + 2 * d_kv) * bytes_per_elem * (n_cp - 1), n_cp)
        return int(b) if b.denominator == 1 else float(b)
    raise ValueError(f"unknown method {method!r}")


def ulysses_breakeven(h, n_kv):
    """Group size above which Ulysses moves fewer bytes than the ring: 1 + h/n_kv."""
    return 1 + Fraction(h, n_kv)


def overlap_min_tokens(F, B, h, n_kv):
    """Smallest per-GPU chunk for which a ring step hides its send.

    Compute 4 n^2 d / F must cover 4 n d_kv / B, i.e. n >= (F/B)(d_kv/d)
    = (F/B)(n_kv/h) tokens.
    """
    return (F / B) * (n_kv / h)


def visible_flops(pairs, d_k, h_q):
    """Attention FLOPs of the visible pairs: 4*d_k per pair per query head."""
    return 4 * int(d_k) * int(h_q) * int(pairs)

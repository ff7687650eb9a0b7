"""Ring-attention oracle: layouts, the per-block partial, the online-softmax fold,
finalisation and brute-force attention, all in numpy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Nothing here is tuned:
each function is the plain definition written out, so that it can be checked
against the pages by eye.  Every input is upcast to float64 exactly as given
(bf16-representable or fp32 values), and all arithmetic is float64.

Conventions shared by every function below:

* ``q`` is ``[h_q][n_q][d_k]``, ``k`` and ``v`` are ``[h_kv][n_k][d_k]``.
* ``q_pos`` and ``k_pos`` are the explicit global token positions of the rows.
* Key j is visible to query i iff ``k_pos[j] <= q_pos[i]`` (causal) or always
  (non-causal).  A query sees itself: with "every earlier token" read strictly,
  position 0 would have nothing to attend to.
* Query head h reads key/value head ``h // (h_q // h_kv)`` (consecutive query
  heads share a key/value head).  The pages give only the ratio of query to
  key/value heads, not the assignment.
* Document masks (packed sequences, Zero to Frontier "Splitting the
  sequence ...": gathering the keys and values makes such masks easy to
  support): when ``q_doc`` and ``k_doc`` give each query and key the id of the
  document it belongs to, a visible key must also be in the query's document.
  Without them every key is in one document.
* Scores are ``scale * q.k`` with ``scale = 1/sqrt(d_k)`` unless given.
* State (m, l, O) is the running maximum, running exp-sum and running
  unnormalised weighted value sum of the online softmax, in natural-log units
  of the scaled score.  An empty row is (-inf, 0, 0).
"""

import math

import numpy as np

LAYOUTS = ("contiguous", "zigzag", "striped")

# Query rows are processed in chunks so that one score matrix never exceeds
# about this many float64 values.  Rows are independent, so chunking the rows
# changes no arithmetic.
_MAX_SCORE_ELEMS = 1 << 24


def default_scale(d_k):
    """Softmax scale 1/sqrt(d_k)."""
    return 1.0 / math.sqrt(d_k)


def positions(T, n_cp, r, layout):
    """Global positions of the tokens rank ``r`` holds, in local order.

    * contiguous: the r-th of n_cp equal runs, ``[r*n, (r+1)*n)`` with
      n = T/n_cp.  The curry-train "What it does" section prints the range
      with closed brackets; the half-open reading is the only one that splits
      the sequence.
    * zigzag: cut T into 2*n_cp equal chunks; rank r holds chunk r followed by
      its mirror chunk 2*n_cp-1-r (Zero to Frontier, "The causal mask
      unbalances the sequence": one chunk from the front, its mirror from the
      back).
    * striped: round-robin, token t goes to rank t mod n_cp (same section,
      after Brandon et al.), so rank r holds r, r+n_cp, r+2*n_cp, ...
    """
    if layout not in LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    if not (0 <= r < n_cp):
        raise ValueError("rank out of range")
    if layout == "contiguous":
        if T % n_cp:
            raise ValueError("T must be divisible by n_cp")
        n = T // n_cp
        return np.arange(r * n, (r + 1) * n, dtype=np.int64)
    if layout == "zigzag":
        if T % (2 * n_cp):
            raise ValueError("T must be divisible by 2*n_cp")
        c = T // (2 * n_cp)
        front = np.arange(r * c, (r + 1) * c, dtype=np.int64)
        back_chunk = 2 * n_cp - 1 - r
        back = np.arange(back_chunk * c, (back_chunk + 1) * c, dtype=np.int64)
        return np.concatenate([front, back])
    # striped
    if T % n_cp:
        raise ValueError("T must be divisible by n_cp")
    return np.arange(r, T, n_cp, dtype=np.int64)


def ring_sources(n_cp, r):
    """Rank whose key/value block rank ``r`` holds at each ring step.

    Each step a GPU sends the block it holds to its right neighbour and
    receives the next one from its left (Zero to Frontier, "Splitting the
    sequence ..."), so at step b rank r holds the block that started on rank
    (r - b) mod n_cp.  Step 0 is the rank's own block.
    """
    return [(r - b) % n_cp for b in range(n_cp)]


def init_state(h_q, n_q, d_k):
    """Empty online-softmax state: m = -inf, l = 0, O = 0."""
    return (
        np.full((h_q, n_q), -np.inf, dtype=np.float64),
        np.zeros((h_q, n_q), dtype=np.float64),
        np.zeros((h_q, n_q, d_k), dtype=np.float64),
    )


def _check(q, k, v, q_pos, k_pos):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    h_q, n_q, d = q.shape
    h_kv, n_k, d2 = k.shape
    if v.shape != k.shape or d2 != d:
        raise ValueError("k and v must be [h_kv][n_k][d_k] with q's d_k")
    if h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    if q_pos.shape != (n_q,) or k_pos.shape != (n_k,):
        raise ValueError("positions must match the row counts")
    return q, k, v, q_pos, k_pos


def _row_chunks(n_q, n_k):
    step = max(1, _MAX_SCORE_ELEMS // max(1, n_k))
    for i0 in range(0, n_q, step):
        yield slice(i0, min(n_q, i0 + step))


def doc_ids(pos, doc_starts):
    """Document id of each global position: the index of the last document
    start at or before it.  ``doc_starts`` are the increasing first positions
    of the packed documents (the first one 0)."""
    starts = np.asarray(doc_starts, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    return np.searchsorted(starts, pos, side="right") - 1


def _visible(q_pos_rows, k_pos, causal, q_doc_rows, k_doc):
    """[rows][n_k] visibility: causal order, and the same document when
    documents are given; None when every key is visible."""
    vis = None
    if causal:
        vis = k_pos[None, :] <= q_pos_rows[:, None]
    if q_doc_rows is not None:
        same = np.asarray(k_doc)[None, :] == np.asarray(q_doc_rows)[:, None]
        vis = same if vis is None else (vis & same)
    return vis


def _docs(q_doc, k_doc, n_q, n_k):
    if (q_doc is None) != (k_doc is None):
        raise ValueError("give both q_doc and k_doc, or neither")
    if q_doc is None:
        return None, None
    q_doc = np.asarray(q_doc, dtype=np.int64)
    k_doc = np.asarray(k_doc, dtype=np.int64)
    if q_doc.shape != (n_q,) or k_doc.shape != (n_k,):
        raise ValueError("document ids must match the row counts")
    return q_doc, k_doc


def block_partial(q, q_pos, k, v, k_pos, scale=None, causal=True, q_doc=None, k_doc=None):
    """Softmax partial of every query against one key/value block.

    For each query head h and query i, over the visible keys j of the block:
    m_b = max_j s_ij, l_b = sum_j exp(s_ij - m_b), O_b = sum_j exp(s_ij - m_b) v_j,
    with s_ij = scale * q_i . k_j.  A row with no visible key gives
    (-inf, 0, 0).  This is the per-block piece of the online softmax
    (Zero to Frontier, "Splitting the sequence ...": running maximum, running
    sum of exponentials, running weighted sum of the values).
    """
    q, k, v, q_pos, k_pos = _check(q, k, v, q_pos, k_pos)
    h_q, n_q, d = q.shape
    h_kv, n_k, _ = k.shape
    q_doc, k_doc = _docs(q_doc, k_doc, n_q, n_k)
    g = h_q // h_kv
    if scale is None:
        scale = default_scale(d)
    m = np.full((h_q, n_q), -np.inf)
    l = np.zeros((h_q, n_q))
    O = np.zeros((h_q, n_q, d))
    if n_q == 0 or n_k == 0:
        return m, l, O
    for h in range(h_q):
        kv = h // g
        for rows in _row_chunks(n_q, n_k):
            s = scale * (q[h, rows] @ k[kv].T)
            visible = _visible(q_pos[rows], k_pos, causal,
                               None if q_doc is None else q_doc[rows], k_doc)
            if visible is not None:
                s = np.where(visible, s, -np.inf)
            mb = s.max(axis=1)
            shift = np.where(np.isfinite(mb), mb, 0.0)
            p = np.exp(s - shift[:, None])  # exp(-inf) == 0 for hidden keys
            m[h, rows] = mb
            l[h, rows] = p.sum(axis=1)
            O[h, rows] = p @ v[kv]
    return m, l, O


def fold(state, partial):
    """Fold a block partial into the running state (the online-softmax rescale).

    m' = max(m, m_b); alpha = exp(m - m'); beta = exp(m_b - m');
    l' = alpha*l + beta*l_b; O' = alpha*O + beta*O_b.  A factor whose own max
    is -inf contributes nothing (it is 0), so an empty row stays
    (-inf, 0, 0) and never turns into NaN.
    """
    m, l, O = state
    mb, lb, Ob = partial
    mn = np.maximum(m, mb)
    with np.errstate(invalid="ignore"):
        alpha = np.where(np.isneginf(m), 0.0, np.exp(m - mn))
        beta = np.where(np.isneginf(mb), 0.0, np.exp(mb - mn))
    return mn, alpha * l + beta * lb, alpha[..., None] * O + beta[..., None] * Ob


def ring_step_ref(q, q_pos, k, v, k_pos, state, scale=None, causal=True, q_doc=None,
                  k_doc=None):
    """One ring step: fold this block's partial into ``state``."""
    return fold(state, block_partial(q, q_pos, k, v, k_pos, scale, causal, q_doc, k_doc))


def finalize(m, l, O):
    """Normalise: out = O / l and lse = m + ln(l) (natural log).

    A row that saw no key (l = 0) cannot occur for causal rank shares, since
    every query's own position is among the keys; it is given out = 0 and
    lse = -inf rather than NaN.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    ok = l > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(ok[..., None], O / np.where(ok, l, 1.0)[..., None], 0.0)
        lse = np.where(ok, m + np.log(np.where(ok, l, 1.0)), -np.inf)
    return out, lse


def ring_forward_ref(q, q_pos, k_blocks, v_blocks, k_pos_blocks, scale=None,
                     causal=True, return_state=False, q_doc=None, k_doc_blocks=None):
    """One rank's forward share: fold every block in the given (ring) order,
    then normalise.  Returns (out, lse) and optionally the final state.  With
    ``q_doc`` and ``k_doc_blocks`` (document ids of the queries and of each
    block's keys) the document mask applies as well."""
    q = np.asarray(q, dtype=np.float64)
    h_q, n_q, d = q.shape
    state = init_state(h_q, n_q, d)
    if k_doc_blocks is None:
        k_doc_blocks = [None] * len(k_blocks)
    for k, v, kp, kd in zip(k_blocks, v_blocks, k_pos_blocks, k_doc_blocks):
        state = ring_step_ref(q, q_pos, k, v, kp, state, scale, causal, q_doc, kd)
    out, lse = finalize(*state)
    if return_state:
        return out, lse, state
    return out, lse


def brute_attention(q, q_pos, k, v, k_pos, scale=None, causal=True, q_doc=None, k_doc=None):
    """Ordinary (non-blockwise) masked softmax attention over all keys at once.

    For each query: lse = log sum_j exp(s_ij) over visible j (computed with the
    row maximum subtracted) and out = sum_j softmax(s)_ij v_j.  Rows with no
    visible key give out = 0 and lse = -inf.
    """
    q, k, v, q_pos, k_pos = _check(q, k, v, q_pos, k_pos)
    h_q, n_q, d = q.shape
    h_kv, n_k, _ = k.shape
    q_doc, k_doc = _docs(q_doc, k_doc, n_q, n_k)
    g = h_q // h_kv
    if scale is None:
        scale = default_scale(d)
    out = np.zeros((h_q, n_q, d))
    lse = np.full((h_q, n_q), -np.inf)
    if n_q == 0 or n_k == 0:
        return out, lse
    for h in range(h_q):
        kv = h // g
        for rows in _row_chunks(n_q, n_k):
            s = scale * (q[h, rows] @ k[kv].T)
            visible = _visible(q_pos[rows], k_pos, causal,
                               None if q_doc is None else q_doc[rows], k_doc)
            if visible is not None:
                s = np.where(visible, s, -np.inf)
            mx = s.max(axis=1)
            has = np.isfinite(mx)
            shift = np.where(has, mx, 0.0)
            e = np.exp(s - shift[:, None])
            tot = e.sum(axis=1)
            with np.errstate(divide="ignore", invalid="ignore"):
                probs = np.where(has[:, None], e / np.where(has, tot, 1.0)[:, None], 0.0)
                lse[h, rows] = np.where(has, shift + np.log(np.where(has, tot, 1.0)), -np.inf)
            out[h, rows] = probs @ v[kv]
    return out, lse

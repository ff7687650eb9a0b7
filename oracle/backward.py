"""Backward of one rank's share: gradients of the attention output with
respect to the local queries and to every key/value block, in numpy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Zero to Frontier, "distributed/context-expert", section "Splitting the
sequence, and the one layer that objects": the backward pass mirrors the
forward.  Each GPU computes, from its own queries, gradients for every key and
value block it sees.  In the all-gather form a reduce-scatter then returns
each block's gradient to its owner.  In the ring the key/value gradients
travel as a second circulating block ("What context parallelism
communicates").  Per block, this is the textbook gradient of softmax attention
written out, using the log-sum-exp the forward returned (over all blocks) so
that every block's probabilities are already normalised:

    s_ij  = scale * q_i . k_j          (visible pairs only)
    p_ij  = exp(s_ij - lse_i)
    dv_j  = sum_i p_ij dout_i
    dp_ij = dout_i . v_j
    D_i   = dout_i . out_i             (= sum_j p_ij dp_ij over every block)
    ds_ij = p_ij (dp_ij - D_i)
    dq_i  = scale * sum_j ds_ij k_j
    dk_j  = scale * sum_i ds_ij q_i

Query head h reads key/value head h // (h_q / h_kv); the key/value gradients
of a shared head sum over the query heads that read it.  A row that sees no
key at all (lse = -inf) contributes nothing.
"""

import numpy as np

from .ring import _check, _row_chunks, default_scale


def backward_prep_ref(out, dout):
    """D_i = dout_i . out_i per query head and row."""
    out = np.asarray(out, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    return (out * dout).sum(axis=-1)


def block_backward_ref(q, q_pos, k, v, k_pos, dout, lse, D, scale=None, causal=True):
    """One key/value block's share of the backward: (dq contribution, dk, dv).

    dq is ``[h_q][n_q][d_k]`` (this block's part; the blocks' parts add up),
    dk and dv are ``[h_kv][n_k][d_k]``.
    """
    q, k, v, q_pos, k_pos = _check(q, k, v, q_pos, k_pos)
    dout = np.asarray(dout, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    h_q, n_q, d = q.shape
    h_kv, n_k, _ = k.shape
    g = h_q // h_kv
    if scale is None:
        scale = default_scale(d)
    dq = np.zeros((h_q, n_q, d))
    dk = np.zeros((h_kv, n_k, d))
    dv = np.zeros((h_kv, n_k, d))
    if n_q == 0 or n_k == 0:
        return dq, dk, dv
    for h in range(h_q):
        kv = h // g
        for rows in _row_chunks(n_q, n_k):
            s = scale * (q[h, rows] @ k[kv].T)
            visible = np.ones(s.shape, dtype=bool)
            if causal:
                visible = k_pos[None, :] <= q_pos[rows, None]
            li = lse[h, rows]
            seen = np.isfinite(li)
            with np.errstate(invalid="ignore", over="ignore"):
                p = np.where(visible & seen[:, None], np.exp(s - np.where(seen, li, 0.0)[:, None]),
                             0.0)
            dp = dout[h, rows] @ v[kv].T
            ds = p * (dp - D[h, rows][:, None])
            dv[kv] += p.T @ dout[h, rows]
            dq[h, rows] = scale * (ds @ k[kv])
            dk[kv] += scale * (ds.T @ q[h, rows])
    return dq, dk, dv


def ring_backward_ref(q, q_pos, k_blocks, v_blocks, k_pos_blocks, out, lse, dout,
                      scale=None, causal=True):
    """The rank share's backward: dq summed over the blocks, and one (dk, dv)
    per block, in the order the blocks were given."""
    D = backward_prep_ref(out, dout)
    q = np.asarray(q, dtype=np.float64)
    dq = np.zeros(q.shape)
    dks, dvs = [], []
    for k, v, kp in zip(k_blocks, v_blocks, k_pos_blocks):
        dq_b, dk, dv = block_backward_ref(q, q_pos, k, v, kp, dout, lse, D, scale, causal)
        dq += dq_b
        dks.append(dk)
        dvs.append(dv)
    return dq, dks, dvs

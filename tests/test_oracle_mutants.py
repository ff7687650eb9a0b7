"""Plant plausible mistakes in the oracle (on the CPU) and check that the
pins catch every one of them: a dropped term, a wrong sign, a wrong index, a
swapped operand, a wrong log base, an off-by-one mask or chunk."""

import math

import numpy as np
import pytest

import oracle
import oracle.counts
import oracle.ring
import pins
import test_oracle_counts as tc
import test_oracle_layouts as tl


def _bp(q, q_pos, k, v, k_pos, scale=None, causal=True, q_doc=None, k_doc=None, mistake=None):
    """The block partial with one planted mistake (these pins use no documents)."""
    assert q_doc is None and k_doc is None
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    q_pos = np.asarray(q_pos); k_pos = np.asarray(k_pos)
    h_q, n_q, d = q.shape
    h_kv, n_k, _ = k.shape
    g = h_q // h_kv
    if scale is None:
        scale = 1.0 if mistake == "no_scale" else 1 / math.sqrt(d)
    m = np.full((h_q, n_q), -np.inf); l = np.zeros((h_q, n_q)); O = np.zeros((h_q, n_q, d))
    if n_q == 0 or n_k == 0:
        return m, l, O
    for h in range(h_q):
        kv = h % h_kv if mistake == "gqa_roundrobin" else h // g
        s = scale * (q[h] @ k[kv].T)
        if causal:
            vis = (k_pos[None, :] < q_pos[:, None]) if mistake == "strict_mask" else (k_pos[None, :] <= q_pos[:, None])
            s = np.where(vis, s, -np.inf)
        mb = s.max(axis=1)
        shift = np.where(np.isfinite(mb), mb, 0.0)
        p = np.exp(s - shift[:, None])
        m[h] = mb
        l[h] = p.sum(axis=1)
        O[h] = p @ (k[kv] if mistake == "k_for_v" else v[kv])
    return m, l, O


def _fold(mistake):
    def f(state, partial):
        m, l, O = state
        mb, lb, Ob = partial
        mn = np.maximum(m, mb)
        with np.errstate(invalid="ignore", over="ignore"):
            a = np.where(np.isneginf(m), 0.0, np.exp(m - mn))
            b = np.where(np.isneginf(mb), 0.0, np.exp(mb - mn))
            if mistake == "no_alpha":
                a = np.where(np.isneginf(m), 0.0, 1.0)
            if mistake == "alpha_sign":
                a = np.where(np.isneginf(m), 0.0, np.exp(mn - m))
            if mistake == "min_not_max":
                mn = np.where(np.isneginf(m), mb, np.where(np.isneginf(mb), m, np.minimum(m, mb)))
                a = np.where(np.isneginf(m), 0.0, np.exp(m - mn))
                b = np.where(np.isneginf(mb), 0.0, np.exp(mb - mn))
        if mistake == "l_not_rescaled":
            return mn, l + b * lb, a[..., None] * O + b[..., None] * Ob
        return mn, a * l + b * lb, a[..., None] * O + b[..., None] * Ob
    return f


def _finalize_log2(m, l, O):
    ok = l > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        return (np.where(ok[..., None], O / np.where(ok, l, 1)[..., None], 0.0),
                np.where(ok, m + np.log2(np.where(ok, l, 1)), -np.inf))


def _positions_zigzag_off_by_one(T, n_cp, r, layout):
    if layout != "zigzag":
        return _orig_positions(T, n_cp, r, layout)
    c = T // (2 * n_cp)
    back = (2 * n_cp - r) % (2 * n_cp)
    return np.concatenate([np.arange(r * c, (r + 1) * c), np.arange(back * c, (back + 1) * c)])


_orig_positions = oracle.ring.positions


def _causal_work_full_diagonal(assignment):
    total = sum(len(c) for c in assignment)
    return [float(sum(a + 1 for a in ch)) for ch in assignment]


def _comm_bytes_ncp(T, d, d_kv, n_cp, method, bytes_per_elem=2):
    n = T // n_cp
    if method == "ulysses":
        return n * (2 * d + 2 * d_kv) * bytes_per_elem * (n_cp - 1) / n_cp
    return n_cp * 2 * n * d_kv * bytes_per_elem


def _breakeven_no_one(h, n_kv):
    return h / n_kv


def _tile_work_any_is_full(q_pos, k_pos, BM, BN, causal=True):
    f = m = s = 0
    for i0 in range(0, len(q_pos), BM):
        for j0 in range(0, len(k_pos), BN):
            vis = np.asarray(k_pos)[j0:j0 + BN][None, :] <= np.asarray(q_pos)[i0:i0 + BM][:, None]
            if vis.any():
                f += 1
            else:
                s += 1
    return f, m, s


def _bp_with(mistake):
    return lambda *a, **kw: _bp(*a, **kw, mistake=mistake)


MUTANTS = {
    "partial_gqa_roundrobin": [("ring", "block_partial", _bp_with("gqa_roundrobin"))],
    "partial_strict_mask": [("ring", "block_partial", _bp_with("strict_mask"))],
    "partial_no_scale": [("ring", "block_partial", _bp_with("no_scale"))],
    "partial_k_for_v": [("ring", "block_partial", _bp_with("k_for_v"))],
    "fold_no_alpha": [("ring", "fold", _fold("no_alpha"))],
    "fold_alpha_sign": [("ring", "fold", _fold("alpha_sign"))],
    "fold_min_not_max": [("ring", "fold", _fold("min_not_max"))],
    "fold_l_not_rescaled": [("ring", "fold", _fold("l_not_rescaled"))],
    "finalize_log2": [("ring", "finalize", _finalize_log2)],
    "zigzag_mirror_off_by_one": [("ring", "positions", _positions_zigzag_off_by_one)],
    "work_diagonal_full": [("counts", "causal_work", _causal_work_full_diagonal)],
    "comm_bytes_n_cp_blocks": [("counts", "cp_comm_bytes", _comm_bytes_ncp)],
    "breakeven_missing_one": [("counts", "ulysses_breakeven", _breakeven_no_one)],
    "tiles_any_is_full": [("counts", "tile_work", _tile_work_any_is_full)],
}

CHECKS = list(pins.ALL_PINS) + [
    tc.test_contiguous_work_matches_pages,
    lambda: tc.test_zigzag_work_is_equal(4),
    tc.test_llama405b_allgather_bytes,
    tc.test_ulysses_breakeven_and_byte_model,
    tc.test_tile_work_brute_small_and_ragged,
    lambda: tc.test_half_blocks_from_tiles_match_pages(4),
    lambda: tl.test_positions_agree_with_chunk_assignment(64, 4),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for mod, attr, fn in MUTANTS[name]:
        monkeypatch.setattr(getattr(oracle, mod), attr, fn)
        monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for check in CHECKS:
        try:
            with np.errstate(all="ignore"):
                check()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(getattr(check, "__name__", "lambda"))
    assert caught, f"mutant {name} passed every pin"

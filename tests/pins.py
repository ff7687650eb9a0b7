"""Pins of the attention oracle against things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
brute force, a library routine, a closed form or an invariant.  They are run
as ordinary tests (tests/test_oracle_attention.py) and, with mistakes planted
in the oracle, as mutation tests (tests/test_oracle_mutants.py), which check
that every plausible mistake is caught by at least one pin.
"""

import math

import numpy as np
import torch

import oracle

TOL = 1e-12


def _rand(rng, shape, amp=1.0):
    return amp * rng.standard_normal(shape)


def _sdpa_ref(q, k, v, causal, scale):
    """Textbook attention from torch (float64, CPU): SDPA output and logsumexp."""
    h_q, h_kv = q.shape[0], k.shape[0]
    g = h_q // h_kv
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(np.repeat(k, g, axis=0))
    vt = torch.from_numpy(np.repeat(v, g, axis=0))
    out = torch.nn.functional.scaled_dot_product_attention(
        qt[None], kt[None], vt[None], is_causal=causal, scale=scale)[0].numpy()
    s = scale * torch.einsum("hid,hjd->hij", qt, kt)
    if causal:
        n_q, n_k = s.shape[1], s.shape[2]
        mask = torch.ones(n_q, n_k, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1).numpy()
    return out, lse


def pin_brute_vs_torch(seed=0):
    """n_cp = 1: causal attention with positions 0..T-1 is textbook attention."""
    rng = np.random.default_rng(seed)
    for h_q, h_kv, T, d in [(4, 4, 37, 16), (6, 2, 64, 8), (4, 1, 33, 32)]:
        q, k, v = _rand(rng, (h_q, T, d)), _rand(rng, (h_kv, T, d)), _rand(rng, (h_kv, T, d))
        pos = np.arange(T)
        scale = 1 / math.sqrt(d)
        for causal in (True, False):
            out, lse = oracle.brute_attention(q, pos, k, v, pos, None, causal)
            ro, rl = _sdpa_ref(q, k, v, causal, scale)
            assert np.abs(out - ro).max() < 1e-12, "brute out vs torch"
            assert np.abs(lse - rl).max() < 1e-12, "brute lse vs torch"


def _layout_case(rng, T, n_cp, layout, h_q, h_kv, d, amp=1.0):
    q = _rand(rng, (h_q, T, d), amp)
    k = _rand(rng, (h_kv, T, d), amp)
    v = _rand(rng, (h_kv, T, d))
    return q, k, v


def pin_ring_vs_brute(seed=1):
    """Ring fold over blocks (ring order and shuffled) equals brute force."""
    rng = np.random.default_rng(seed)
    for layout in oracle.LAYOUTS:
        for (h_q, h_kv) in [(4, 4), (4, 2), (6, 1)]:
            T, n_cp, d = 48, 4, 8
            q, k, v = _layout_case(rng, T, n_cp, layout, h_q, h_kv, d)
            for r in range(n_cp):
                qp = oracle.positions(T, n_cp, r, layout)
                srcs = oracle.ring_sources(n_cp, r)
                orders = [srcs, list(rng.permutation(srcs))]
                allk = np.concatenate([oracle.positions(T, n_cp, s, layout) for s in srcs])
                bo, bl = oracle.brute_attention(q[:, qp], qp, k[:, allk], v[:, allk], allk)
                for order in orders:
                    kps = [oracle.positions(T, n_cp, s, layout) for s in order]
                    out, lse = oracle.ring_forward_ref(
                        q[:, qp], qp, [k[:, p] for p in kps], [v[:, p] for p in kps], kps)
                    assert np.abs(out - bo).max() < TOL, (layout, h_q, h_kv, r, "out")
                    assert np.abs(lse - bl).max() < TOL, (layout, h_q, h_kv, r, "lse")


def pin_layout_invariance(seed=2):
    """Every layout's rank shares, put back at their global positions, give
    ordinary causal attention over the whole sequence (via torch)."""
    rng = np.random.default_rng(seed)
    T, n_cp, h_q, h_kv, d = 64, 4, 4, 2, 16
    q, k, v = _layout_case(rng, T, n_cp, None, h_q, h_kv, d)
    ref_out, ref_lse = _sdpa_ref(q, k, v, True, 1 / math.sqrt(d))
    for layout in oracle.LAYOUTS:
        g_out = np.full_like(ref_out, np.nan)
        g_lse = np.full_like(ref_lse, np.nan)
        for r in range(n_cp):
            qp = oracle.positions(T, n_cp, r, layout)
            kps = [oracle.positions(T, n_cp, s, layout) for s in oracle.ring_sources(n_cp, r)]
            out, lse = oracle.ring_forward_ref(q[:, qp], qp, [k[:, p] for p in kps],
                                               [v[:, p] for p in kps], kps)
            g_out[:, qp] = out
            g_lse[:, qp] = lse
        assert not np.isnan(g_out).any(), layout
        assert np.abs(g_out - ref_out).max() < 1e-12, layout
        assert np.abs(g_lse - ref_lse).max() < 1e-12, layout


def pin_closed_forms(seed=3):
    """Cases with a closed form.

    * K = 0: every visible score is 0, so out_i is the mean of V over keys at
      positions <= q_pos_i and lse_i = ln(number of such keys).
    * V constant: out is that constant.
    * A query at position 0 sees only key 0: out = V[0], lse = scale q.k_0.
    """
    rng = np.random.default_rng(seed)
    T, n_cp, h_q, h_kv, d = 40, 4, 4, 2, 8
    g = h_q // h_kv
    for layout in oracle.LAYOUTS:
        r = 1
        qp = oracle.positions(T, n_cp, r, layout)
        kps = [oracle.positions(T, n_cp, s, layout) for s in oracle.ring_sources(n_cp, r)]
        q = _rand(rng, (h_q, T, d))[:, qp]
        v = _rand(rng, (h_kv, T, d))
        zeros = np.zeros((h_kv, T, d))
        out, lse = oracle.ring_forward_ref(q, qp, [zeros[:, p] for p in kps], [v[:, p] for p in kps], kps)
        for h in range(h_q):
            for i, p in enumerate(qp):
                assert abs(lse[h, i] - math.log(p + 1)) < 1e-12
                assert np.abs(out[h, i] - v[h // g, :p + 1].mean(axis=0)).max() < 1e-12
        kfull = _rand(rng, (h_kv, T, d))
        const = np.full((h_kv, T, d), 0.375)
        out, _ = oracle.ring_forward_ref(q, qp, [kfull[:, p] for p in kps], [const[:, p] for p in kps], kps)
        assert np.abs(out - 0.375).max() < 1e-12
    # position-0 query
    qp = np.array([0, 5])
    kp = np.arange(8)
    q = _rand(rng, (h_q, 2, d))
    k = _rand(rng, (h_kv, 8, d))
    v = _rand(rng, (h_kv, 8, d))
    scale = 0.3
    out, lse = oracle.ring_forward_ref(q, qp, [k[:, :3], k[:, 3:]], [v[:, :3], v[:, 3:]], [kp[:3], kp[3:]], scale)
    for h in range(h_q):
        assert np.abs(out[h, 0] - v[h // g, 0]).max() < 1e-12
        assert abs(lse[h, 0] - scale * float(q[h, 0] @ k[h // g, 0])) < 1e-12


def pin_gqa_equals_duplicated_mha(seed=4):
    """Query head h reads KV head h // (h_q/h_kv): same as MHA with each KV
    head repeated for its group of consecutive query heads."""
    rng = np.random.default_rng(seed)
    T, n_cp, h_q, h_kv, d = 32, 2, 6, 3, 8
    q = _rand(rng, (h_q, T, d))
    k = _rand(rng, (h_kv, T, d))
    v = _rand(rng, (h_kv, T, d))
    kd, vd = np.repeat(k, 2, axis=0), np.repeat(v, 2, axis=0)
    qp = oracle.positions(T, n_cp, 1, "zigzag")
    kps = [oracle.positions(T, n_cp, s, "zigzag") for s in oracle.ring_sources(n_cp, 1)]
    a = oracle.ring_forward_ref(q[:, qp], qp, [k[:, p] for p in kps], [v[:, p] for p in kps], kps)
    b = oracle.ring_forward_ref(q[:, qp], qp, [kd[:, p] for p in kps], [vd[:, p] for p in kps], kps)
    assert np.abs(a[0] - b[0]).max() < 1e-13 and np.abs(a[1] - b[1]).max() < 1e-13
    # and the head mapping is consecutive groups, not round-robin:
    # changing KV head 0 must change query heads 0 and 1 only.
    k2 = k.copy()
    k2[0] += rng.standard_normal(k2[0].shape)  # not a constant: softmax ignores per-row shifts
    c = oracle.ring_forward_ref(q[:, qp], qp, [k2[:, p] for p in kps], [v[:, p] for p in kps], kps)
    changed = [bool(np.abs(c[0][h] - a[0][h]).max() > 1e-9) for h in range(h_q)]
    assert changed == [True, True, False, False, False, False], changed


def pin_checkpoint_resume(seed=5):
    """The state after any prefix of steps is a complete checkpoint: folding
    the rest from a saved copy gives the uninterrupted result bit for bit."""
    rng = np.random.default_rng(seed)
    T, n_cp, h_q, h_kv, d = 48, 4, 4, 2, 8
    q = _rand(rng, (h_q, T, d))
    k = _rand(rng, (h_kv, T, d))
    v = _rand(rng, (h_kv, T, d))
    r = 2
    qp = oracle.positions(T, n_cp, r, "striped")
    kps = [oracle.positions(T, n_cp, s, "striped") for s in oracle.ring_sources(n_cp, r)]
    full = oracle.init_state(h_q, len(qp), d)
    for p in kps:
        full = oracle.ring_step_ref(q[:, qp], qp, k[:, p], v[:, p], p, full)
    for cut in range(n_cp + 1):
        st = oracle.init_state(h_q, len(qp), d)
        for p in kps[:cut]:
            st = oracle.ring_step_ref(q[:, qp], qp, k[:, p], v[:, p], p, st)
        saved = tuple(np.array(x, copy=True) for x in st)
        for p in kps[cut:]:
            saved = oracle.ring_step_ref(q[:, qp], qp, k[:, p], v[:, p], p, saved)
        for a, b in zip(saved, full):
            assert np.array_equal(a, b)


def pin_empty_rows(seed=6):
    """A block wholly in the future leaves the state bit-identical, an empty
    state finalises to out = 0 and lse = -inf, and nothing becomes NaN."""
    rng = np.random.default_rng(seed)
    h_q, h_kv, d = 2, 1, 8
    q = _rand(rng, (h_q, 4, d))
    qp = np.array([0, 1, 2, 3])
    k = _rand(rng, (h_kv, 4, d))
    v = _rand(rng, (h_kv, 4, d))
    st = oracle.init_state(h_q, 4, d)
    st1 = oracle.ring_step_ref(q, qp, k, v, np.array([10, 11, 12, 13]), st)
    for a, b in zip(st, st1):
        assert np.array_equal(a, b)
    out, lse = oracle.finalize(*st1)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    st2 = oracle.ring_step_ref(q, qp, k, v, np.array([0, 1, 2, 3]), st1)
    st3 = oracle.ring_step_ref(q, qp, k, v, np.array([10, 11, 12, 13]), st2)
    for a, b in zip(st2, st3):
        assert np.array_equal(a, b)
        assert not np.isnan(a).any()
    # a row that sees only some keys of a block
    st4 = oracle.ring_step_ref(q, qp, k, v, np.array([2, 3, 4, 5]), oracle.init_state(h_q, 4, d))
    assert np.all(np.isneginf(st4[0][:, :2])) and np.all(st4[1][:, :2] == 0)
    assert np.all(np.isfinite(st4[0][:, 2:]))


def pin_scale_and_noncausal(seed=7):
    """An explicit scale is used as given, and non-causal attention sees every
    key whatever the positions."""
    rng = np.random.default_rng(seed)
    h, n, d = 2, 10, 4
    q, k, v = _rand(rng, (h, n, d)), _rand(rng, (h, n, d)), _rand(rng, (h, n, d))
    pos = np.arange(n)
    ro, rl = _sdpa_ref(q, k, v, False, 0.7)
    rev = pos[::-1].copy()
    out, lse = oracle.ring_forward_ref(q, rev, [k[:, :4], k[:, 4:]], [v[:, :4], v[:, 4:]],
                                       [pos[:4], pos[4:]], scale=0.7, causal=False)
    assert np.abs(out - ro).max() < 1e-12 and np.abs(lse - rl).max() < 1e-12


def pin_extreme_scores(seed=8):
    """Scores spanning thousands of units (far beyond exp's range) still give
    finite results equal to brute force: the fold must rescale towards the
    running maximum, never away from it."""
    rng = np.random.default_rng(seed)
    T, n_cp, h_q, h_kv, d = 32, 4, 2, 1, 8
    q = _rand(rng, (h_q, T, d), 40.0)
    k = _rand(rng, (h_kv, T, d), 40.0)
    v = _rand(rng, (h_kv, T, d))
    for layout in oracle.LAYOUTS:
        r = n_cp - 1
        qp = oracle.positions(T, n_cp, r, layout)
        srcs = oracle.ring_sources(n_cp, r)
        kps = [oracle.positions(T, n_cp, s, layout) for s in srcs]
        allk = np.concatenate(kps)
        out, lse = oracle.ring_forward_ref(q[:, qp], qp, [k[:, p] for p in kps], [v[:, p] for p in kps], kps)
        bo, bl = oracle.brute_attention(q[:, qp], qp, k[:, allk], v[:, allk], allk)
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
        assert np.abs(out - bo).max() < 1e-9 and np.abs(lse - bl).max() < 1e-9 * np.abs(bl).max()


ALL_PINS = [
    pin_extreme_scores,
    pin_brute_vs_torch,
    pin_ring_vs_brute,
    pin_layout_invariance,
    pin_closed_forms,
    pin_gqa_equals_duplicated_mha,
    pin_checkpoint_resume,
    pin_empty_rows,
    pin_scale_and_noncausal,
]

"""The oracle's document mask (packed sequences; Zero to Frontier,
"distributed/context-expert", "Splitting the sequence, and the one layer that
objects": gathering the keys and values makes arbitrary masks such as
document masks easy to support) against torch per document, brute force,
invariants and brute-counted tiles, plus planted mistakes that these pins
must catch."""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.counts
import oracle.ring
import ring_attention_rank_amd.layouts as L
import synth


def _rand(rng, shape):
    return rng.standard_normal(shape)


def _sdpa(q, k, v, scale):
    """Textbook causal attention from torch (float64, CPU) on one document."""
    g = q.shape[0] // k.shape[0]
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(np.repeat(k, g, axis=0))
    vt = torch.from_numpy(np.repeat(v, g, axis=0))
    out = torch.nn.functional.scaled_dot_product_attention(
        qt[None], kt[None], vt[None], is_causal=True, scale=scale)[0].numpy()
    s = scale * torch.einsum("hid,hjd->hij", qt, kt)
    n = s.shape[1]
    s = s.masked_fill(~torch.ones(n, n, dtype=torch.bool).tril(), float("-inf"))
    return out, torch.logsumexp(s, dim=-1).numpy()


def _docs(T, rng, lo, hi):
    starts = [0]
    while True:
        nxt = starts[-1] + int(rng.integers(lo, hi + 1))
        if nxt >= T:
            return np.asarray(starts)
        starts.append(nxt)


def test_doc_ids():
    starts = np.array([0, 5, 9])
    assert oracle.doc_ids(np.arange(12), starts).tolist() == [0] * 5 + [1] * 4 + [2] * 3


def test_docs_equal_torch_per_document():
    """The whole sequence on one rank: each document is textbook causal
    attention over its own tokens (torch SDPA), independent of the others."""
    rng = np.random.default_rng(11)
    for h_q, h_kv, T, d in [(4, 4, 96, 8), (6, 2, 80, 16), (4, 1, 64, 8)]:
        q, k, v = _rand(rng, (h_q, T, d)), _rand(rng, (h_kv, T, d)), _rand(rng, (h_kv, T, d))
        starts = _docs(T, rng, 1, 24)
        pos = np.arange(T)
        ids = oracle.doc_ids(pos, starts)
        out, lse = oracle.ring_forward_ref(q, pos, [k], [v], [pos], q_doc=ids, k_doc_blocks=[ids])
        bounds = list(starts) + [T]
        for a, b in zip(bounds[:-1], bounds[1:]):
            ro, rl = _sdpa(q[:, a:b], k[:, a:b], v[:, a:b], 1 / math.sqrt(d))
            assert np.abs(out[:, a:b] - ro).max() < 1e-12
            assert np.abs(lse[:, a:b] - rl).max() < 1e-12


@pytest.mark.parametrize("layout", oracle.LAYOUTS)
def test_docs_blockwise_equals_brute_any_order(layout):
    """The fold over blocks (ring order and shuffled) equals brute force over
    all keys at once, with documents."""
    rng = np.random.default_rng(12)
    T, n_cp, d = 64, 4, 8
    for h_q, h_kv in [(4, 4), (4, 1)]:
        q, k, v = _rand(rng, (h_q, T, d)), _rand(rng, (h_kv, T, d)), _rand(rng, (h_kv, T, d))
        starts = _docs(T, rng, 1, 20)
        for r in (0, n_cp - 1):
            qp = oracle.positions(T, n_cp, r, layout)
            srcs = oracle.ring_sources(n_cp, r)
            allk = np.concatenate([oracle.positions(T, n_cp, s, layout) for s in srcs])
            qd, kd_all = oracle.doc_ids(qp, starts), oracle.doc_ids(allk, starts)
            bo, bl = oracle.brute_attention(q[:, qp], qp, k[:, allk], v[:, allk], allk,
                                            q_doc=qd, k_doc=kd_all)
            for order in (srcs, list(rng.permutation(srcs))):
                kps = [oracle.positions(T, n_cp, s, layout) for s in order]
                out, lse = oracle.ring_forward_ref(
                    q[:, qp], qp, [k[:, p] for p in kps], [v[:, p] for p in kps], kps,
                    q_doc=qd, k_doc_blocks=[oracle.doc_ids(p, starts) for p in kps])
                assert np.abs(out - bo).max() < 1e-12
                assert np.abs(lse - bl).max() < 1e-12


def test_one_document_is_plain_causal():
    rng = np.random.default_rng(13)
    T, n_cp, d = 48, 4, 8
    q, k, v = _rand(rng, (4, T, d)), _rand(rng, (2, T, d)), _rand(rng, (2, T, d))
    qp = oracle.positions(T, n_cp, 1, "zigzag")
    kps = [oracle.positions(T, n_cp, s, "zigzag") for s in oracle.ring_sources(n_cp, 1)]
    zero = np.zeros(T, dtype=np.int64)
    a = oracle.ring_forward_ref(q[:, qp], qp, [k[:, p] for p in kps], [v[:, p] for p in kps], kps)
    b = oracle.ring_forward_ref(q[:, qp], qp, [k[:, p] for p in kps], [v[:, p] for p in kps], kps,
                                q_doc=zero[qp], k_doc_blocks=[zero[p] for p in kps])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_single_token_documents():
    """A document of one token: the query sees only itself, so out is its own
    value row and lse its own scaled score."""
    rng = np.random.default_rng(14)
    T, d = 16, 8
    q, k, v = _rand(rng, (2, T, d)), _rand(rng, (2, T, d)), _rand(rng, (2, T, d))
    pos = np.arange(T)
    starts = np.array([0, 3, 4, 9, 10])  # documents of one token at 3 and 9
    ids = oracle.doc_ids(pos, starts)
    out, lse = oracle.ring_forward_ref(q, pos, [k], [v], [pos], q_doc=ids, k_doc_blocks=[ids])
    for t in (3, 9):
        assert np.abs(out[:, t] - v[:, t]).max() < 1e-15
        assert np.abs(lse[:, t] - np.einsum("hd,hd->h", q[:, t], k[:, t]) / math.sqrt(d)).max() < 1e-12


def test_tile_work_with_documents_brute_count():
    rng = np.random.default_rng(15)
    for layout in oracle.LAYOUTS:
        T, n_cp = 96, 2
        starts = _docs(T, rng, 3, 30)
        qp = oracle.positions(T, n_cp, 1, layout)
        kp = oracle.positions(T, n_cp, 0, layout)
        qd, kd = oracle.doc_ids(qp, starts), oracle.doc_ids(kp, starts)
        for BM, BN in [(8, 8), (4, 16), (16, 4)]:
            full = masked = skipped = 0
            for i0 in range(0, qp.size, BM):
                for j0 in range(0, kp.size, BN):
                    cnt = tot = 0
                    for i in range(i0, min(i0 + BM, qp.size)):
                        for j in range(j0, min(j0 + BN, kp.size)):
                            tot += 1
                            cnt += int(kp[j] <= qp[i] and kd[j] == qd[i])
                    full += cnt == tot
                    skipped += cnt == 0
                    masked += 0 < cnt < tot
            assert oracle.tile_work(qp, kp, BM, BN, q_doc=qd, k_doc=kd) == (full, masked, skipped)


def test_document_start_form_matches_ids():
    """The kernels take each query's document start as a lower bound on the
    key positions it sees; for packed documents that is the same visibility
    as 'same document and not later', pair by pair."""
    rng = np.random.default_rng(16)
    for layout in oracle.LAYOUTS:
        T, n_cp = 64, 4
        starts = _docs(T, rng, 1, 16)
        qp = oracle.positions(T, n_cp, 2, layout)
        kp = np.concatenate([oracle.positions(T, n_cp, s, layout) for s in range(n_cp)])
        lo = L.document_start_of(qp, starts)
        by_bound = (kp[None, :] <= qp[:, None]) & (kp[None, :] >= lo[:, None])
        qd, kd = oracle.doc_ids(qp, starts), oracle.doc_ids(kp, starts)
        by_ids = (kp[None, :] <= qp[:, None]) & (kd[None, :] == qd[:, None])
        assert np.array_equal(by_bound, by_ids)
        assert np.all(np.diff(lo) >= 0) and np.all(lo <= qp)


def test_synth_document_starts():
    s = synth.document_starts(131072, 1004)
    assert s[0] == 0 and np.all(np.diff(s) > 0) and s[-1] < 131072
    lens = np.diff(np.append(s, 131072))
    assert lens[:-1].min() >= 512 and lens.max() <= 32768
    assert np.array_equal(s, synth.document_starts(131072, 1004))


# ---- planted mistakes: each must fail at least one of the pins above ------

def _planted_partial(mistake):
    real = oracle.ring.block_partial

    def bp(q, q_pos, k, v, k_pos, scale=None, causal=True, q_doc=None, k_doc=None):
        if q_doc is not None:
            q_doc, k_doc = np.asarray(q_doc), np.asarray(k_doc)
            if mistake == "ignore_docs":
                q_doc = k_doc = None
            elif mistake == "merge_neighbours":   # document 2i+1 also sees document 2i
                q_doc, k_doc = q_doc // 2, k_doc // 2
            elif mistake == "key_ids_off_by_one":  # a query sees the next document's keys
                k_doc = k_doc + 1
        return real(q, q_pos, k, v, k_pos, scale, causal, q_doc, k_doc)

    return bp


@pytest.mark.parametrize("mistake", ["ignore_docs", "merge_neighbours", "key_ids_off_by_one"])
def test_planted_document_mistakes_are_caught(monkeypatch, mistake):
    monkeypatch.setattr(oracle.ring, "block_partial", _planted_partial(mistake))
    caught = 0
    for pin in (test_docs_equal_torch_per_document, test_single_token_documents):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, mistake

"""Pins of the backward oracle against things other than itself: torch's
autograd of an independently written float64 attention, central finite
differences of the forward oracle, and the sum rule of the value gradient."""

import numpy as np
import pytest
import torch

import oracle


def _share(rng, layout, n_cp, r, T, h_q, h_kv, d):
    q_pos = oracle.positions(T, n_cp, r, layout)
    srcs = oracle.ring_sources(n_cp, r)
    k_pos = [oracle.positions(T, n_cp, s, layout) for s in srcs]
    n = T // n_cp
    q = rng.standard_normal((h_q, n, d))
    kb = [rng.standard_normal((h_kv, n, d)) for _ in srcs]
    vb = [rng.standard_normal((h_kv, n, d)) for _ in srcs]
    return q, q_pos, kb, vb, k_pos


def _torch_grads(q, q_pos, kb, vb, k_pos, dout, causal=True):
    """Autograd of plain masked softmax attention over the concatenated blocks."""
    h_q, n_q, d = q.shape
    h_kv = kb[0].shape[0]
    g = h_q // h_kv
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = [torch.tensor(k, dtype=torch.float64, requires_grad=True) for k in kb]
    tv = [torch.tensor(v, dtype=torch.float64, requires_grad=True) for v in vb]
    K = torch.cat(tk, dim=1)
    V = torch.cat(tv, dim=1)
    kp = torch.tensor(np.concatenate(k_pos))
    qp = torch.tensor(q_pos)
    mask = kp[None, :] <= qp[:, None] if causal else torch.ones(n_q, len(kp), dtype=torch.bool)
    Kh = K.repeat_interleave(g, dim=0)
    Vh = V.repeat_interleave(g, dim=0)
    s = (tq @ Kh.transpose(1, 2)) / np.sqrt(d)
    s = s.masked_fill(~mask[None], float("-inf"))
    out = torch.softmax(s, dim=-1) @ Vh
    (out * torch.tensor(dout)).sum().backward()
    return (tq.grad.numpy(), [t.grad.numpy() for t in tk], [t.grad.numpy() for t in tv],
            out.detach().numpy())


@pytest.mark.parametrize("layout,n_cp,r", [("contiguous", 4, 2), ("zigzag", 4, 1), ("striped", 4, 3)])
@pytest.mark.parametrize("h_q,h_kv", [(2, 2), (4, 2)])
def test_matches_torch_autograd(layout, n_cp, r, h_q, h_kv):
    rng = np.random.default_rng(hash((layout, n_cp, r, h_q)) % 2**32)
    q, q_pos, kb, vb, k_pos = _share(rng, layout, n_cp, r, 64, h_q, h_kv, 8)
    dout = rng.standard_normal(q.shape)
    out, lse = oracle.ring_forward_ref(q, q_pos, kb, vb, k_pos)
    dq, dks, dvs = oracle.ring_backward_ref(q, q_pos, kb, vb, k_pos, out, lse, dout)
    tdq, tdk, tdv, tout = _torch_grads(q, q_pos, kb, vb, k_pos, dout)
    assert np.abs(out - tout).max() < 1e-12
    assert np.abs(dq - tdq).max() < 1e-11
    for b in range(n_cp):
        assert np.abs(dks[b] - tdk[b]).max() < 1e-11
        assert np.abs(dvs[b] - tdv[b]).max() < 1e-11


def test_noncausal_and_scale_sign():
    rng = np.random.default_rng(5)
    q, q_pos, kb, vb, k_pos = _share(rng, "zigzag", 2, 0, 32, 2, 1, 4)
    dout = rng.standard_normal(q.shape)
    out, lse = oracle.ring_forward_ref(q, q_pos, kb, vb, k_pos, causal=False)
    dq, dks, dvs = oracle.ring_backward_ref(q, q_pos, kb, vb, k_pos, out, lse, dout, causal=False)
    tdq, tdk, tdv, _ = _torch_grads(q, q_pos, kb, vb, k_pos, dout, causal=False)
    assert np.abs(dq - tdq).max() < 1e-11
    assert max(np.abs(a - b).max() for a, b in zip(dks, tdk)) < 1e-11


def test_finite_differences():
    """Central differences of L = sum(dout * out) through the forward oracle."""
    rng = np.random.default_rng(7)
    q, q_pos, kb, vb, k_pos = _share(rng, "zigzag", 2, 1, 16, 2, 1, 4)
    dout = rng.standard_normal(q.shape)
    out, lse = oracle.ring_forward_ref(q, q_pos, kb, vb, k_pos)
    dq, dks, dvs = oracle.ring_backward_ref(q, q_pos, kb, vb, k_pos, out, lse, dout)

    def loss(q_, kb_, vb_):
        o, _ = oracle.ring_forward_ref(q_, q_pos, kb_, vb_, k_pos)
        return float((o * dout).sum())

    eps = 1e-6
    for (h, i, c) in [(0, 0, 0), (1, 5, 3), (0, 7, 2)]:
        qp, qm = q.copy(), q.copy()
        qp[h, i, c] += eps
        qm[h, i, c] -= eps
        assert abs((loss(qp, kb, vb) - loss(qm, kb, vb)) / (2 * eps) - dq[h, i, c]) < 1e-7
    for b, (h, j, c) in [(0, (0, 1, 1)), (1, (0, 6, 0))]:
        for which, grads in (("k", dks), ("v", dvs)):
            src = kb if which == "k" else vb
            plus = [x.copy() for x in src]
            minus = [x.copy() for x in src]
            plus[b][h, j, c] += eps
            minus[b][h, j, c] -= eps
            if which == "k":
                num = (loss(q, plus, vb) - loss(q, minus, vb)) / (2 * eps)
            else:
                num = (loss(q, kb, plus) - loss(q, kb, minus)) / (2 * eps)
            assert abs(num - grads[b][h, j, c]) < 1e-7, (which, b, h, j, c)


def test_value_gradient_sum_rule():
    """Every row's probabilities sum to 1 over all blocks, so the value
    gradients of all blocks sum to the output gradients of the query heads
    that read them; and each row's score gradients sum to 0, so the query
    gradient is orthogonal to a key shift common to all keys."""
    rng = np.random.default_rng(9)
    q, q_pos, kb, vb, k_pos = _share(rng, "striped", 4, 2, 64, 4, 2, 8)
    dout = rng.standard_normal(q.shape)
    out, lse = oracle.ring_forward_ref(q, q_pos, kb, vb, k_pos)
    dq, dks, dvs = oracle.ring_backward_ref(q, q_pos, kb, vb, k_pos, out, lse, dout)
    tot_dv = sum(dv.sum(axis=1) for dv in dvs)            # [h_kv][d]
    tot_do = dout.reshape(2, 2, *dout.shape[1:]).sum(axis=(1, 2))
    assert np.abs(tot_dv - tot_do).max() < 1e-10
    # Shifting every key by the same vector c moves all visible scores of a
    # row by the same amount, so no softmax changes; hence the gradient with
    # respect to such a shift, sum_j dk_j over all blocks (= scale * sum_i
    # (sum_j ds_ij) q_i), is zero.
    c = rng.standard_normal(8)
    shifted = [k + c for k in kb]
    out2, _ = oracle.ring_forward_ref(q, q_pos, shifted, vb, k_pos)
    assert np.abs(out2 - out).max() < 1e-10
    tot_dk = sum(dk.sum(axis=1) for dk in dks)
    assert np.abs(tot_dk).max() < 1e-10

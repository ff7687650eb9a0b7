"""Parity of the backward (ra_backward_prep + ra_backward_step, bfloat16 with
d_k = 128) with the float64 oracle: element by element at reduced sizes with
ragged tails, GQA and every layout; sampled rows and sum rules at full size.

Both sides get the same inputs: q, k, v, dout (bfloat16 values), and the
forward's out and lse from the oracle, rounded to float32 (the library's
input types).

Tolerance, per element.  Against the exact product, the MFMA path (bfloat16,
d_k = 128) rounds two things to bfloat16 before an MFMA reads them: p (for
dv) and ds (for dq and dk); everything else is float32.  Rounding to nearest
moves a value by at most 2^-8 of itself, so

    |dq_gpu - dq| <= scale (2^-8 |ds| + e p (A + |D|)) @ |k| + 1e-6

(dk with q in place of k, dv with 2^-8 p @ |dout|), where
A = |dout| @ |v|^T bounds the float32 error of dp, and e = 1e-4 covers the
float32 errors of s, the exponential, dp and D (each under about 1e-5 of
these magnitudes at d_k = 128).  The plain kernels for the other shapes
(float32 inputs, bfloat16 with d_k = 64) round nothing to bfloat16: there
the 2^-8 terms are 0.
"""

import numpy as np
import pytest
import torch

import oracle
import ring_attention_rank_amd as ra
import synth
from gpu_util import Share, sample_rows
from test_gpu_parity import _custom_share

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

U_BF16 = 2.0 ** -8
E_F32 = 1e-4
ABS = 1e-6


def fwd_inputs(sh, dout_seed_case=None):
    """Oracle forward (out, lse) rounded to float32, and seeded dout."""
    out, lse = sh.oracle()
    out32 = out.astype(np.float32)
    lse32 = lse.astype(np.float32)
    dout = synth.case_dout(dout_seed_case or sh.case, sh.q_pos)
    return out32, lse32, dout


def run_gpu(sh, out32, lse32, dout, blocks=None):
    idx = range(len(sh.gk)) if blocks is None else blocks
    g = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    dt = torch.bfloat16 if sh.case.dtype == "bf16" else torch.float32
    dq, dks, dvs = ra.backward(sh.gq, sh.gq_pos, [sh.gk[i] for i in idx], [sh.gv[i] for i in idx],
                               [sh.gk_pos[i] for i in idx], g(out32), g(lse32), g(dout).to(dt),
                               causal=sh.case.causal)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), [x.cpu().numpy() for x in dks], [x.cpu().numpy() for x in dvs]


def rounding(case):
    """Relative rounding of p and ds before the products: bf16 on the MFMA
    path, none on the plain kernels."""
    return U_BF16 if (case.dtype == "bf16" and case.d_k == 128) else 0.0


def bounds(q, q_pos, k, v, k_pos, dout, lse, D, causal, u=U_BF16):
    """Per-element error bounds (dq, dk, dv) for one block (see the module
    docstring); ``u`` is the relative rounding of p and ds."""
    h_q, n_q, d = q.shape
    h_kv, n_k, _ = k.shape
    g = h_q // h_kv
    scale = 1.0 / np.sqrt(d)
    bq = np.zeros((h_q, n_q, d))
    bk = np.zeros((h_kv, n_k, d))
    bv = np.zeros((h_kv, n_k, d))
    for h in range(h_q):
        kv = h // g
        s = scale * (q[h].astype(np.float64) @ k[kv].T.astype(np.float64))
        vis = (k_pos[None, :] <= q_pos[:, None]) if causal else np.ones(s.shape, bool)
        seen = np.isfinite(lse[h])
        vis &= seen[:, None]
        with np.errstate(over="ignore", invalid="ignore"):
            p = np.where(vis, np.exp(s - np.where(seen, lse[h], 0.0)[:, None]), 0.0)
        dp = dout[h].astype(np.float64) @ v[kv].T.astype(np.float64)
        A = np.abs(dout[h]).astype(np.float64) @ np.abs(v[kv]).T.astype(np.float64)
        ads = np.abs(p * (dp - D[h][:, None]))
        m = u * ads + E_F32 * p * (A + np.abs(D[h])[:, None])
        bq[h] = scale * (m @ np.abs(k[kv]))
        bk[kv] += scale * (m.T @ np.abs(q[h]))
        bv[kv] += (u + E_F32) * (p.T @ np.abs(dout[h]))
    return bq, bk, bv


def check_close(got, ref, bound, label):
    err = np.abs(got.astype(np.float64) - ref)
    lim = bound + ABS
    bad = err > lim
    assert np.all(np.isfinite(got)), f"{label}: non-finite values"
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{label}: {bad.sum()} elements out of bound; worst at {i}: "
                             f"got {got[i]}, oracle {ref[i]}, bound {lim[i]}")


def check_share(sh, label):
    print(f"[backward] {label}", flush=True)
    out32, lse32, dout = fwd_inputs(sh)
    dq, dks, dvs = run_gpu(sh, out32, lse32, dout)
    causal = sh.case.causal
    rq, rks, rvs = oracle.ring_backward_ref(sh.q, sh.q_pos, sh.k, sh.v, sh.k_pos, out32, lse32,
                                            dout, causal=causal)
    D = oracle.backward_prep_ref(out32, dout)
    bq_tot = np.zeros(rq.shape)
    for b in range(len(sh.k)):
        bq, bk, bv = bounds(sh.q, sh.q_pos, sh.k[b], sh.v[b], sh.k_pos[b], dout, lse32, D, causal,
                            rounding(sh.case))
        bq_tot += bq
        check_close(dks[b], rks[b], bk, f"{label} dk block {b}")
        check_close(dvs[b], rvs[b], bv, f"{label} dv block {b}")
    check_close(dq, rq, bq_tot, f"{label} dq")


@pytest.mark.parametrize("name,T,n_cp,rank", [
    ("llama8b_gqa_zigzag", 4096, 4, 1),
    ("llama70b_stage_share", 8192, 16, 15),
    ("llama405b_stage_share", 16384, 16, 0),
    ("million_striped_mha", 16384, 64, 5),
])
def test_reduced_configs(name, T, n_cp, rank):
    sh = Share(synth.case_by_name(name), rank, T=T, n_cp=n_cp).to_gpu()
    check_share(sh, f"{name}@T{T}/r{rank}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n_q,n_k,h_q,h_kv", [(517, 129, 4, 2), (300, 200, 4, 2), (1, 70, 3, 3),
                                              (64, 64, 2, 1), (130, 1, 2, 2)])
def test_ragged_and_small(n_q, n_k, h_q, h_kv, causal):
    rng = np.random.default_rng(n_q * 7 + n_k + 5)
    sh = _custom_share(rng, "bf16", 128, h_q, h_kv, n_q, n_k, 3, causal=causal)
    check_share(sh, f"ragged nq{n_q} nk{n_k} h{h_q}/{h_kv} causal={causal}")


def test_rows_that_see_no_key():
    """Queries placed before every key have lse = -inf: their dq is zero and
    they add nothing to dk and dv."""
    rng = np.random.default_rng(5)
    sh = _custom_share(rng, "bf16", 128, 4, 2, 200, 150, 2)
    # the first 70 queries take positions 0..69 and every key moves past them
    # (the 71st distinct position is at least 70, so positions stay increasing)
    sh.q_pos = sh.q_pos.copy()
    sh.q_pos[:70] = np.arange(70)
    sh.k_pos = [p + 70 for p in sh.k_pos]
    sh.to_gpu()
    out32, lse32, dout = fwd_inputs(sh)
    assert np.all(np.isneginf(lse32[:, :70]))
    check_share(sh, "rows that see no key")
    dq, _, _ = run_gpu(sh, out32, lse32, dout)
    assert np.all(dq[:, :70] == 0.0)


def test_empty_sides():
    rng = np.random.default_rng(9)
    sh = _custom_share(rng, "bf16", 128, 4, 2, 96, 80, 1)
    out32, lse32, dout = fwd_inputs(sh)
    g = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    gdout = g(dout).to(torch.bfloat16)
    delta = ra.backward_prep(g(out32), gdout)
    # no keys: dq keeps what it held
    dq = torch.full(sh.gq.shape, 0.25, dtype=torch.float32, device="cuda")
    k0 = sh.gk[0][:, :0].contiguous()
    kp0 = sh.gk_pos[0][:0].contiguous()
    dk, dv = ra.backward_step(sh.gq, sh.gq_pos, k0, k0, kp0, gdout, g(lse32), delta, dq)
    torch.cuda.synchronize()
    assert torch.all(dq == 0.25) and dk.numel() == 0 and dv.numel() == 0
    # no queries: dk and dv keep what they held
    q0 = sh.gq[:, :0].contiguous()
    e = torch.empty((4, 0), dtype=torch.float32, device="cuda")
    dq0 = torch.empty((4, 0, 128), dtype=torch.float32, device="cuda")
    dk = torch.full(sh.gk[0].shape, 7.0, dtype=torch.float32, device="cuda")
    dv = torch.full(sh.gk[0].shape, 7.0, dtype=torch.float32, device="cuda")
    ra.backward_step(q0, sh.gq_pos[:0].contiguous(), sh.gk[0], sh.gv[0], sh.gk_pos[0],
                     gdout[:, :0].contiguous(), e, e, dq0, dk, dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 7.0) and torch.all(dv == 7.0)


@pytest.mark.parametrize("h_q,h_kv,n_k", [(4, 2, 200), (16, 1, 256)])
def test_dk_dv_accumulate(h_q, h_kv, n_k):
    """dk and dv are added to what the caller passes (the travelling
    gradients of the ring), with and without the head-group split."""
    rng = np.random.default_rng(h_q * 31 + n_k)
    sh = _custom_share(rng, "bf16", 128, h_q, h_kv, 160, n_k, 1)
    out32, lse32, dout = fwd_inputs(sh)
    g = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    gdout = g(dout).to(torch.bfloat16)
    delta = ra.backward_prep(g(out32), gdout)
    p = ra._problem_from(sh.gq, sh.gk[0], True, None)
    print(f"[backward] accumulate h{h_q}/{h_kv} nk{n_k} workspace "
          f"{ra.backward_workspace_bytes(p)}", flush=True)
    dq = torch.zeros(sh.gq.shape, dtype=torch.float32, device="cuda")
    dk0, dv0 = ra.backward_step(sh.gq, sh.gq_pos, sh.gk[0], sh.gv[0], sh.gk_pos[0], gdout,
                                g(lse32), delta, dq)
    base_k = torch.from_numpy(rng.standard_normal(dk0.shape).astype(np.float32)).cuda()
    base_v = torch.from_numpy(rng.standard_normal(dv0.shape).astype(np.float32)).cuda()
    dk, dv = base_k.clone(), base_v.clone()
    ra.backward_step(sh.gq, sh.gq_pos, sh.gk[0], sh.gv[0], sh.gk_pos[0], gdout, g(lse32), delta,
                     torch.zeros_like(dq), dk, dv)
    torch.cuda.synchronize()
    # one float32 addition per element, in the kernel as here
    assert torch.equal(dk, base_k + dk0) and torch.equal(dv, base_v + dv0)


@pytest.mark.parametrize("dtype,d_k", [("f32", 64), ("f32", 128), ("bf16", 64)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n_q,n_k,h_q,h_kv", [(300, 200, 4, 2), (1, 70, 3, 3), (130, 1, 2, 2)])
def test_plain_kernels(dtype, d_k, n_q, n_k, h_q, h_kv, causal):
    """The shapes outside the MFMA path run the plain float32 kernels."""
    rng = np.random.default_rng(n_q * 11 + n_k + d_k)
    sh = _custom_share(rng, dtype, d_k, h_q, h_kv, n_q, n_k, 3, causal=causal)
    check_share(sh, f"plain {dtype} d{d_k} nq{n_q} nk{n_k} h{h_q}/{h_kv} causal={causal}")


def test_plain_kernels_full_tile_share():
    """A reduced ring share of the fp32 workload through the plain kernels."""
    sh = Share(synth.case_by_name("tiny_f32_contiguous"), 2).to_gpu()
    check_share(sh, "tiny_f32_contiguous r2")


def test_unsupported_shapes_refused():
    rng = np.random.default_rng(3)
    sh = _custom_share(rng, "bf16", 128, 2, 2, 64, 64, 1)
    q96 = torch.zeros((2, 64, 96), dtype=torch.bfloat16, device="cuda")
    z = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    dq = torch.zeros(q96.shape, dtype=torch.float32, device="cuda")
    k96 = torch.zeros((2, 64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ra.RAError, match="sizes"):
        ra.backward_step(q96, sh.gq_pos, k96, k96, sh.gk_pos[0], q96, z, z, dq)


@pytest.mark.parametrize("name", ["llama405b_stage_share", "llama70b_stage_share",
                                  "llama8b_gqa_zigzag", "million_striped_mha"])
def test_full_size_sampled(name):
    """A share at full size (405B stage: 8192 queries, 16 heads, 16 blocks of
    8192 keys; 70B stage: 8 heads; 8B: 32 query heads on 8 key/value heads,
    4 blocks; striped MHA: 8 heads, 64 blocks), in the launch configuration
    the benchmark times.  Sampled rows' dq against the oracle (those rows get
    the oracle's out and lse; the other rows take the library's forward, which
    only the sum rules below use).  Sum rules over all blocks: per key/value
    head, sum_j dv_j = sum over the group's heads of sum_i dout_i (the
    probabilities of each row sum to one), and sum_i q_i . dq_i =
    sum_j k_j . dk_j (both equal sum_ij ds_ij s_ij)."""
    case = synth.case_by_name(name)
    sh = Share(case, 0).to_gpu()
    print(f"[backward] {name} full size", flush=True)
    out, lse, _, _ = ra.forward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    rows = sample_rows(sh.q_pos, n_rand=24, seed=4)
    ro, rl = sh.oracle(rows)
    ro32, rl32 = ro.astype(np.float32), rl.astype(np.float32)
    out[:, torch.from_numpy(rows).cuda()] = torch.from_numpy(ro32).cuda()
    lse[:, torch.from_numpy(rows).cuda()] = torch.from_numpy(rl32).cuda()
    dout = synth.case_dout(case, sh.q_pos)
    gdout = torch.from_numpy(dout).cuda().to(torch.bfloat16)
    dq, dks, dvs = ra.backward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos, out, lse, gdout)
    torch.cuda.synchronize()

    # sampled rows against the oracle
    q_s = sh.q[:, rows]
    rq, _, _ = oracle.ring_backward_ref(q_s, sh.q_pos[rows], sh.k, sh.v, sh.k_pos, ro32, rl32,
                                        dout[:, rows])
    D = oracle.backward_prep_ref(ro32, dout[:, rows])
    bq = np.zeros(rq.shape)
    for b in range(len(sh.k)):
        bq += bounds(q_s, sh.q_pos[rows], sh.k[b], sh.v[b], sh.k_pos[b], dout[:, rows], rl32, D,
                     True)[0]
    check_close(dq[:, rows].cpu().numpy(), rq, bq, "full-size dq rows")

    # sum_j dv_j = sum_i dout_i: p of a row sums to one up to the float32 lse
    # (1e-5 here) and the bfloat16 rounding of each p
    sum_dv = sum(x.double().sum(dim=1) for x in dvs).cpu().numpy()  # [h_kv][d]
    grouped = dout.astype(np.float64).reshape(case.h_kv, case.h_q // case.h_kv, -1, case.d_k)
    want = grouped.sum(axis=(1, 2))
    lim = (U_BF16 + 1e-4) * np.abs(grouped).sum(axis=(1, 2))
    assert np.all(np.abs(sum_dv - want) <= lim), float(np.abs(sum_dv - want).max())

    # sum_i q_i . dq_i = sum_j k_j . dk_j, over the group's heads and all blocks
    lhs = float((sh.gq.double() * dq.double()).sum())
    rhs = float(sum((k.double() * x.double()).sum() for k, x in zip(sh.gk, dks)))
    mag = float((sh.gq.double().abs() * dq.double().abs()).sum())
    assert abs(lhs - rhs) <= 1e-3 * mag, (lhs, rhs, mag)


def _share_inputs(sh):
    out32, lse32, dout = fwd_inputs(sh)
    dt = torch.bfloat16 if sh.case.dtype == "bf16" else torch.float32
    g = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return g(out32), g(lse32), g(dout).to(dt)


@pytest.mark.parametrize("side", [True, False])
@pytest.mark.parametrize("which", ["405b", "ragged", "f32"])
def test_whole_share_equals_block_steps(which, side):
    """ra_backward_share (every block in one call, dk/dv on a side stream)
    gives bit for bit what the block-by-block ra_backward_step loop gives:
    same kernels, same order of additions into dq (its first block's kernel
    writes dq where the loop adds to zeros, and dk, dv are written where the
    loop adds them to zeros: the same values)."""
    if which == "405b":
        sh = Share(synth.case_by_name("llama405b_stage_share"), 0, T=16384, n_cp=16).to_gpu()
    elif which == "ragged":
        sh = _custom_share(np.random.default_rng(21), "bf16", 128, 4, 2, 517, 129, 3)
    else:
        sh = _custom_share(np.random.default_rng(22), "f32", 64, 4, 2, 300, 200, 3)
    print(f"[backward] whole share {which} side={side}", flush=True)
    out, lse, dout = _share_inputs(sh)
    a_dq, a_dks, a_dvs = ra.backward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos, out, lse, dout,
                                     causal=sh.case.causal)
    f = ra.BackwardShare(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos, causal=sh.case.causal,
                         side=side)
    # garbage in the outputs first: the call overwrites them
    f.dq.fill_(3.0)
    for t in f.dks + f.dvs:
        t.fill_(-5.0)
    for rep in range(2):
        b_dq, b_dks, b_dvs = f(out, lse, dout)
        torch.cuda.synchronize()
        assert torch.equal(a_dq, b_dq), rep
        for x, y in zip(a_dks + a_dvs, b_dks + b_dvs):
            assert torch.equal(x, y), rep


@pytest.mark.parametrize("h_q,h_kv", [(256, 1), (256, 256)])
def test_max_heads(h_q, h_kv):
    """256 query heads: the head-group split of the dk/dv grid with one
    key/value head, and no split with one query head per key/value head."""
    rng = np.random.default_rng(300 + h_kv)
    sh = _custom_share(rng, "bf16", 128, h_q, h_kv, 130, 96, 2)
    check_share(sh, f"max heads {h_q}/{h_kv}")

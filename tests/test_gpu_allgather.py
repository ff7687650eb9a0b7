"""Parity of the all-gather form (ra_forward_allgather: every key/value block
resident, one launch for bf16 d_k = 128, or two side by side where a launch
has one to two work units per compute unit) with the float64 oracle: element
by element at reduced sizes, sampled rows at full size, tile counters bit
exact, the result independent of the block order."""

import numpy as np
import pytest
import torch

import ring_attention_rank_amd as ra
import synth
from gpu_util import TOL, Share, max_err, sample_rows
from test_gpu_parity import _custom_share, compare

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_allgather(sh, order=None):
    idx = list(range(len(sh.gk))) if order is None else list(order)
    out, lse, work = ra.forward_allgather(sh.gq, sh.gq_pos, [sh.gk[i] for i in idx],
                                          [sh.gv[i] for i in idx], [sh.gk_pos[i] for i in idx],
                                          causal=sh.case.causal)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), work.cpu().numpy()


def tiles(sh):
    dt = torch.float32 if sh.case.dtype == "f32" else torch.bfloat16
    return ra.tile_shape(ra.problem(1, 1, sh.case.h_q, sh.case.h_kv, sh.case.d_k, dt))


def check(sh, label):
    print(f"[allgather] {label}", flush=True)
    out, lse, work = run_allgather(sh)
    ro, rl = sh.oracle()
    compare(out, lse, ro, rl, TOL[sh.case.dtype], label)
    assert list(work) == list(sh.tile_work(*tiles(sh))), label


@pytest.mark.parametrize("name,T,n_cp,rank", [
    ("tiny_f32_contiguous", 1024, 4, 2),
    ("llama8b_gqa_zigzag", 4096, 4, 1),
    ("llama70b_stage_share", 8192, 16, 15),
    ("llama405b_stage_share", 8192, 16, 0),
    ("million_striped_mha", 16384, 64, 5),
])
def test_reduced_configs(name, T, n_cp, rank):
    sh = Share(synth.case_by_name(name), rank, T=T, n_cp=n_cp).to_gpu()
    check(sh, f"{name}@T{T}/r{rank}")


@pytest.mark.parametrize("dtype,d_k", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged(dtype, d_k, causal):
    rng = np.random.default_rng(11 + d_k)
    sh = _custom_share(rng, dtype, d_k, 3, 1, 517, 129, 3, causal=causal)
    check(sh, f"ragged {dtype} d{d_k} causal={causal}")


def test_matches_ring_and_is_order_independent():
    sh = Share(synth.case_by_name("llama8b_gqa_zigzag"), 2, T=4096, n_cp=4).to_gpu()
    a_out, a_lse, a_work = run_allgather(sh)
    b_out, b_lse, b_work = run_allgather(sh, order=[3, 1, 0, 2])
    r_out, r_lse, r_work, _ = ra.forward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    torch.cuda.synchronize()
    tol = TOL["bf16"]
    assert max_err(a_out, b_out) <= tol["out"] and max_err(a_lse, b_lse) <= tol["lse"]
    assert max_err(a_out, r_out.cpu().numpy()) <= tol["out"]
    assert max_err(a_lse, r_lse.cpu().numpy()) <= tol["lse"]
    assert list(a_work) == list(b_work) == list(r_work.cpu().numpy())


@pytest.mark.parametrize("n_q,n_k,n_cp", [(2000, 300, 7), (2048, 256, 2)])
def test_two_chains(n_q, n_k, n_cp):
    """One to two work units per compute unit: two one-group launches side by
    side (even and odd blocks, two partial states in the workspace, merged at
    the end), against the oracle, tile counts exact, and within the bound of
    the same blocks in another order."""
    rng = np.random.default_rng(3 * n_q + n_cp)
    sh = _custom_share(rng, "bf16", 128, 32, 8, n_q, n_k, n_cp)
    p = ra.problem(n_q, n_k, 32, 8, 128, torch.bfloat16)
    assert ra.allgather_workspace_bytes(p) > 0  # the two partial states
    check(sh, f"two chains nq{n_q} nk{n_k} ncp{n_cp}")
    a = run_allgather(sh)
    b = run_allgather(sh, order=list(reversed(range(n_cp))))
    compare(a[0], a[1], b[0].astype(np.float64), b[1].astype(np.float64), TOL["bf16"],
            "two chains, blocks reversed")
    assert list(a[2]) == list(b[2])


@pytest.mark.parametrize("name", ["llama405b_stage_share", "llama70b_stage_share",
                                  "million_striped_mha"])
def test_full_size_sampled(name):
    case = synth.case_by_name(name)
    sh = Share(case, 0).to_gpu()
    print(f"[allgather] {name} full size", flush=True)
    out, lse, work = ra.forward_allgather(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    rows = sample_rows(sh.q_pos, seed=5)
    ro, rl = sh.oracle(rows)
    idx = torch.from_numpy(rows).cuda()
    eo = max_err(out[:, idx].cpu().numpy(), ro)
    el = max_err(lse[:, idx].cpu().numpy(), rl)
    print(f"[allgather] {name}: out err {eo:.3e} lse err {el:.3e}", flush=True)
    assert eo <= TOL[case.dtype]["out"] and el <= TOL[case.dtype]["lse"]
    assert list(work.cpu().numpy()) == list(sh.tile_work(*tiles(sh)))

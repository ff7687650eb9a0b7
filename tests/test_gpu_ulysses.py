"""The Ulysses local share on the same kernels: full-sequence causal attention
for the rank's h / n_cp query heads (one block of all T keys, positions
0..T-1; Zero to Frontier, "distributed/context-expert", section "Ulysses,
splitting by heads instead").  Element-wise parity at reduced sizes, sampled
rows at full size, tile counters bit exact, ring and all-gather entry points
alike."""

import numpy as np
import pytest
import torch

import ring_attention_rank_amd as ra
import synth
from gpu_util import TOL, Share, max_err, sample_rows
from test_gpu_parity import compare

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def tiles(case):
    return ra.tile_shape(ra.problem(1, 1, case.h_q, case.h_kv, case.d_k, torch.bfloat16))


@pytest.mark.parametrize("name", ["llama8b_ulysses_share", "llama405b_ulysses_share"])
def test_reduced(name):
    case = synth.case_by_name(name)
    sh = Share(case, 0, T=4096, n_cp=1).to_gpu()
    print(f"[ulysses] {name}@T4096", flush=True)
    ro, rl = sh.oracle()
    out, lse, work, staged = ra.forward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    torch.cuda.synchronize()
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, TOL["bf16"], name)
    assert list(work.cpu().numpy()) == list(sh.tile_work(*tiles(sh.case)))
    assert staged == 0
    out2, lse2, work2 = ra.forward_allgather(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    torch.cuda.synchronize()
    compare(out2.cpu().numpy(), lse2.cpu().numpy(), ro, rl, TOL["bf16"], name + " allgather")
    assert list(work2.cpu().numpy()) == list(work.cpu().numpy())


@pytest.mark.parametrize("name", ["llama8b_ulysses_share", "llama405b_ulysses_share"])
def test_full_size_sampled(name):
    case = synth.case_by_name(name)
    sh = Share(case, 0).to_gpu()
    print(f"[ulysses] {name} full size", flush=True)
    out, lse, work, _ = ra.forward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    rows = sample_rows(sh.q_pos, seed=9)
    ro, rl = sh.oracle(rows)
    idx = torch.from_numpy(rows).cuda()
    eo = max_err(out[:, idx].cpu().numpy(), ro)
    el = max_err(lse[:, idx].cpu().numpy(), rl)
    print(f"[ulysses] {name}: out err {eo:.3e} lse err {el:.3e}", flush=True)
    assert eo <= TOL["bf16"]["out"] and el <= TOL["bf16"]["lse"]
    assert list(work.cpu().numpy()) == list(sh.tile_work(*tiles(case)))

"""The five rank-share workloads at full size, in the launch configuration the
benchmark times (ra_forward with side-stream staging): sampled rows against
the oracle, every row finite, tile counters bit exact, staged bytes exact."""

import numpy as np
import pytest
import torch

import ring_attention_rank_amd as ra
import synth
from gpu_util import TOL, Share, max_err, sample_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _run(name, rank):
    case = synth.case_by_name(name)
    print(f"[fullsize] {name} rank {rank}: building inputs", flush=True)
    sh = Share(case, rank).to_gpu()
    print(f"[fullsize] {name} rank {rank}: ra_forward", flush=True)
    out, lse, work, staged = ra.forward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    rows = sample_rows(sh.q_pos, seed=rank)
    print(f"[fullsize] {name} rank {rank}: oracle on {len(rows)} rows", flush=True)
    ro, rl = sh.oracle(rows)
    go = out[:, torch.from_numpy(rows).cuda()].cpu().numpy()
    gl = lse[:, torch.from_numpy(rows).cuda()].cpu().numpy()
    tol = TOL[case.dtype]
    eo, el = max_err(go, ro), max_err(gl, rl)
    print(f"[fullsize] {name} rank {rank}: out err {eo:.3e} lse err {el:.3e}", flush=True)
    assert eo <= tol["out"] and el <= tol["lse"]
    bm, bn = ra.tile_shape(ra.problem(1, 1, case.h_q, case.h_kv, case.d_k, torch.bfloat16))
    assert list(work.cpu().numpy()) == list(sh.tile_work(bm, bn))
    assert staged == sh.staged_bytes()
    return sh, staged


@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_llama8b_gqa_zigzag(rank):
    _run("llama8b_gqa_zigzag", rank)


def test_llama70b_stage_share():
    _run("llama70b_stage_share", 0)


def test_llama405b_stage_share():
    sh, staged = _run("llama405b_stage_share", 0)
    # the ring delivers the other 15 blocks: 62,914,560 bytes, the pages' "63 MB"
    assert staged == 62_914_560


def test_million_striped_mha():
    _run("million_striped_mha", 0)

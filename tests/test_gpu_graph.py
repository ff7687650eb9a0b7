"""ra_forward captured in a HIP graph (ra.ForwardGraph): every replay, with
eager GPU work and synchronisation between replays, gives bit for bit the
eager result, and a replay after the inputs are changed in place gives the
eager result on the new inputs."""

import pytest
import torch

import ring_attention_rank_amd as ra
import synth
from gpu_util import Share

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def test_replays_equal_eager_and_follow_inputs():
    sh = Share(synth.case_by_name("llama405b_stage_share"), 3, T=8192, n_cp=8).to_gpu()
    args = (sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    eager = ra.Forward(*args)
    ref_out, ref_lse = [t.clone() for t in eager()]
    torch.cuda.synchronize()
    g = ra.ForwardGraph(*args)
    for i in range(3):
        g.out.zero_()
        g.lse.zero_()
        torch.cuda.synchronize()
        out, lse = g()
        torch.cuda.synchronize()
        print(f"[graph] replay {i}", flush=True)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), i
        eager()  # other GPU work between replays
        torch.cuda.synchronize()
    # inputs refreshed in place: the replay reads the new values
    sh.gv[2].mul_(-0.5)
    sh.gq.mul_(0.75)
    torch.cuda.synchronize()
    new_out, new_lse = [t.clone() for t in eager()]
    torch.cuda.synchronize()
    assert not torch.equal(new_out, ref_out)
    out, lse = g()
    torch.cuda.synchronize()
    assert torch.equal(out, new_out) and torch.equal(lse, new_lse)

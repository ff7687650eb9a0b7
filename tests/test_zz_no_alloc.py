"""ra_forward_noalloc against ra_forward: the same ring forward with the
library's fixed per-device workspace instead of the caller's, called twice in
a row (the second call smaller, so it runs on what the first one left in the
array).  Same kernels, same launch order: the results must be identical."""

import numpy as np
import pytest
import torch

import ring_attention_rank_amd as ra
import synth
from gpu_util import Share

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _both(sh):
    out, lse, work, staged = ra.forward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    o2 = torch.full_like(out, float("nan"))
    l2 = torch.full_like(lse, float("nan"))
    w2 = torch.full((3,), -1, dtype=torch.int64, device="cuda")
    st2 = ra.forward_noalloc(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos, o2, l2, w2)
    torch.cuda.synchronize()
    return (out, lse, work, staged), (o2, l2, w2, st2)


@pytest.mark.parametrize("first,second", [
    (("llama8b_gqa_zigzag", 1, 16384, 4), ("llama405b_stage_share", 0, 16384, 8)),
])
def test_noalloc_matches_forward_twice(first, second):
    sizes = []
    for name, rank, T, n_cp in (first, second):
        print(f"[noalloc] {name} rank {rank} T={T} n_cp={n_cp}", flush=True)
        sh = Share(synth.case_by_name(name), rank, T=T, n_cp=n_cp).to_gpu()
        need = ra.workspace_bytes(ra._problem_from(sh.gq, sh.gk[0], True, None))
        assert 0 < need <= ra.NOALLOC_MAX_BYTES
        sizes.append(need)
        (o1, l1, w1, s1), (o2, l2, w2, s2) = _both(sh)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), name
        assert torch.equal(w1, w2) and s1 == s2, name
        assert not np.isnan(o2.cpu().numpy()).any()
    assert sizes[1] < sizes[0]  # the second call runs on a smaller input


def test_noalloc_full_8b_share():
    """The largest share of the size table, the full 8B one: ra_forward's own
    workspace would not fit the array, the no-alloc form's (one state, two
    slots) does, and it gives ra_forward's bits (ra_forward's two blocks per
    launch are bit for bit one launch per block)."""
    print("[noalloc] llama8b_gqa_zigzag full share rank 0", flush=True)
    sh = Share(synth.case_by_name("llama8b_gqa_zigzag"), 0).to_gpu()
    need = ra.workspace_bytes(ra._problem_from(sh.gq, sh.gk[0], True, None))
    assert need > ra.NOALLOC_MAX_BYTES
    (o1, l1, w1, s1), (o2, l2, w2, s2) = _both(sh)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(w1, w2) and s1 == s2


def test_noalloc_refuses_what_does_not_fit():
    """A share whose workspace exceeds the fixed array is refused before any
    work: out and lse keep their contents."""
    h_q, n_q, d = 64, 8192, 128  # state alone: 64 * 8192 * 130 floats > 256 MiB
    q = torch.zeros((h_q, n_q, d), dtype=torch.bfloat16, device="cuda")
    qp = torch.arange(n_q, dtype=torch.int32, device="cuda")
    k = torch.zeros((1, 64, d), dtype=torch.bfloat16, device="cuda")
    kp = torch.arange(64, dtype=torch.int32, device="cuda")
    out = torch.full((h_q, n_q, d), 7.0, device="cuda")
    lse = torch.full((h_q, n_q), 7.0, device="cuda")
    with pytest.raises(ra.RAError) as e:
        ra.forward_noalloc(q, qp, [k], [k], [kp], out, lse)
    assert e.value.status == -5  # RA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())

"""Concurrent against serialized execution: the ring forward (two half
launches per step on two streams, or two chains of launches, blocks staged
on a third) and the whole-share backward (dq and dk/dv kernels on two
streams) give the same bits
when the runtime serializes every kernel and copy (AMD_SERIALIZE_KERNEL=3,
AMD_SERIALIZE_COPY=3, HIP_LAUNCH_BLOCKING=1, in a child process).  A missing
wait between the streams would let a kernel read a slot or a partial result
early in the concurrent run and differ from the serialized one."""

import hashlib
import json
import os
import subprocess
import sys

import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import ring_attention_rank_amd as ra  # noqa: E402
import synth  # noqa: E402
from gpu_util import Share  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def digests(full=False):
    """Hashes of the forward's out and lse and of the backward's dq, dk, dv
    for a reduced 70B stage share (16 blocks of 1024 keys, 8 q / 1 kv heads),
    or for the full one (16 blocks of 8192 keys: the ring forward and the
    all-gather form as two chains of launches on two streams, merged at the
    end)."""
    sh = (Share(synth.case_by_name("llama70b_stage_share"), 0).to_gpu() if full else
          Share(synth.case_by_name("llama70b_stage_share"), 0, T=16384, n_cp=16).to_gpu())
    fwd = ra.Forward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    out, lse = fwd()
    g = torch.Generator(device="cuda").manual_seed(7)
    dout = torch.randn(sh.gq.shape, generator=g, device="cuda").to(torch.bfloat16)
    bwd = ra.BackwardShare(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos, side=True)
    dq, dks, dvs = bwd(out, lse, dout)
    torch.cuda.synchronize()
    h = lambda ts: hashlib.sha256(b"".join(t.cpu().numpy().tobytes() for t in ts)).hexdigest()
    res = {"out": h([out]), "lse": h([lse]), "dq": h([dq]), "dk": h(dks), "dv": h(dvs)}
    if full:  # the all-gather form as two chains on two streams
        ao, al, _ = ra.forward_allgather(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
        torch.cuda.synchronize()
        res["allgather"] = h([ao, al])
    return res


@pytest.mark.parametrize("full", [False, True])
def test_serialized_run_gives_the_same_bits(full):
    here = digests(full)
    env = dict(os.environ, AMD_SERIALIZE_KERNEL="3", AMD_SERIALIZE_COPY="3",
               HIP_LAUNCH_BLOCKING="1")
    print(f"[serialized] child run (full={full})", flush=True)
    r = subprocess.run([sys.executable, os.path.abspath(__file__)] + (["full"] if full else []),
                       env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    there = json.loads(r.stdout.strip().splitlines()[-1])
    assert here == there


if __name__ == "__main__":
    print(json.dumps(digests(len(sys.argv) > 1 and sys.argv[1] == "full")), flush=True)

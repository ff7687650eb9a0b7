"""Parity of the HIP path (through the C ABI) with the float64 oracle, at
sizes the oracle finishes in seconds: element by element, tile counters bit
exact, staged bytes exact.  Edge cases: ragged tiles, empty blocks, rows that
see nothing, non-causal, explicit scale, both dtypes and head widths."""

import numpy as np
import pytest
import torch

import oracle
import ring_attention_rank_amd as ra
import synth
from gpu_util import TOL, Share, max_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_forward(sh, side=True):
    out, lse, work, staged = ra.forward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos,
                                        causal=sh.case.causal, side=side)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), work.cpu().numpy(), staged


def compare(out, lse, ro, rl, tol, label):
    """Element-wise parity; rows that see no key at all must be out = 0 and
    lse = -inf on both sides."""
    out, lse = np.asarray(out), np.asarray(lse)
    empty = np.isneginf(rl)
    assert not np.isnan(out).any() and not np.isnan(lse).any(), label
    assert np.array_equal(np.isneginf(lse), empty), label
    assert np.all(out[empty] == 0) and np.isfinite(out).all(), label
    eo, el = max_err(out, ro), max_err(lse[~empty], rl[~empty])
    assert eo <= tol["out"], f"{label}: out max-abs {eo}"
    assert el <= tol["lse"], f"{label}: lse max-abs {el}"
    return eo, el


def check_share(sh, label):
    print(f"[parity] {label}: T={sh.case.T} n_cp={sh.case.n_cp} rank={sh.rank} "
          f"h={sh.case.h_q}/{sh.case.h_kv} d={sh.case.d_k} {sh.case.dtype}", flush=True)
    out, lse, work, staged = run_forward(sh)
    ro, rl = sh.oracle()
    eo, el = compare(out, lse, ro, rl, TOL[sh.case.dtype], label)
    bm, bn = ra.tile_shape(ra.problem(1, 1, sh.case.h_q, sh.case.h_kv, sh.case.d_k,
                                      torch.float32 if sh.case.dtype == "f32" else torch.bfloat16))
    assert list(work) == list(sh.tile_work(bm, bn)), label
    assert staged == sh.staged_bytes()
    return eo, el


def test_tiny_f32_contiguous_full_size():
    case = synth.case_by_name("tiny_f32_contiguous")
    sh = Share(case, 2).to_gpu()
    check_share(sh, case.name)


@pytest.mark.parametrize("name,T,n_cp,ranks", [
    ("llama8b_gqa_zigzag", 4096, 4, (0, 1, 2, 3)),
    ("llama70b_stage_share", 8192, 16, (0, 15)),
    ("llama405b_stage_share", 8192, 16, (0, 7)),
    ("million_striped_mha", 8192, 16, (0, 15)),
    ("million_striped_mha", 16384, 64, (3,)),
])
def test_reduced_configs(name, T, n_cp, ranks):
    case = synth.case_by_name(name)
    for r in ranks:
        sh = Share(case, r, T=T, n_cp=n_cp).to_gpu()
        check_share(sh, f"{name}@T{T}/r{r}")


def _custom_share(rng, dtype, d_k, h_q, h_kv, n_q, n_k, n_cp, causal=True):
    """Random strictly increasing positions, ragged sizes, blocks in order."""
    case = synth.Case("custom", T=0, n_cp=n_cp, layout="custom", ranks=(0,), h_q=h_q,
                      h_kv=h_kv, d_k=d_k, dtype=dtype, seed=77, causal=causal)
    sh = Share.__new__(Share)
    sh.case, sh.rank = case, 0
    span = 4 * (n_q + n_k * n_cp) + 10
    sh.q_pos = np.sort(rng.choice(span, n_q, replace=False)).astype(np.int64)
    sh.k_pos = [np.sort(rng.choice(span, n_k, replace=False)).astype(np.int64) for _ in range(n_cp)]
    sh.sources = list(range(n_cp))
    bf = dtype == "bf16"
    q = rng.standard_normal((h_q, n_q, d_k)).astype(np.float32)
    sh.q = synth.round_to_bf16(q) if bf else q
    sh.k, sh.v = [], []
    for _ in range(n_cp):
        k = rng.standard_normal((h_kv, n_k, d_k)).astype(np.float32)
        v = rng.standard_normal((h_kv, n_k, d_k)).astype(np.float32)
        sh.k.append(synth.round_to_bf16(k) if bf else k)
        sh.v.append(synth.round_to_bf16(v) if bf else v)
    return sh.to_gpu()


@pytest.mark.parametrize("dtype,d_k", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("n_q,n_k,h_q,h_kv", [(300, 200, 4, 2), (64, 64, 2, 1), (1, 70, 3, 3),
                                              (517, 129, 2, 2)])
def test_ragged_and_small(dtype, d_k, n_q, n_k, h_q, h_kv):
    rng = np.random.default_rng(n_q * 7 + n_k)
    sh = _custom_share(rng, dtype, d_k, h_q, h_kv, n_q, n_k, 3)
    check_share(sh, f"ragged {dtype} d{d_k} nq{n_q} nk{n_k}")


@pytest.mark.parametrize("n_q,h_q,h_kv,causal", [(1000, 128, 8, True), (1024, 128, 1, False),
                                                 (2048, 64, 64, True)])
def test_one_group_workgroups(n_q, h_q, h_kv, causal):
    """Launches of at least two tile pairs x heads per compute unit (512 on
    MI355X) run one 4-wave group per workgroup instead of the two-group
    ping-pong; the same parity, ragged last tile included."""
    rng = np.random.default_rng(n_q + h_q)
    sh = _custom_share(rng, "bf16", 128, h_q, h_kv, n_q, 160, 2, causal=causal)
    n_pairs = ((n_q + 127) // 128 + 1) // 2
    assert n_pairs * h_q >= 2 * torch.cuda.get_device_properties(0).multi_processor_count
    check_share(sh, f"one group nq{n_q} h{h_q}/{h_kv} causal={causal}")
    ro, rl = sh.oracle()
    out, lse, _ = ra.forward_allgather(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos, causal=causal)
    compare(out.cpu(), lse.cpu(), ro, rl, TOL["bf16"], "one group all-gather")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noncausal(dtype):
    rng = np.random.default_rng(11)
    sh = _custom_share(rng, dtype, 128, 4, 1, 200, 100, 3, causal=False)
    check_share(sh, f"noncausal {dtype}")


def test_explicit_scale():
    rng = np.random.default_rng(12)
    sh = _custom_share(rng, "bf16", 128, 2, 1, 128, 128, 2)
    out, lse, _, _ = ra.forward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos, scale=0.05)
    ro, rl = oracle.ring_forward_ref(sh.q, sh.q_pos, sh.k, sh.v, sh.k_pos, scale=0.05)
    compare(out.cpu(), lse.cpu(), ro, rl, TOL["bf16"], "explicit scale")


def _chains(h_q, n_q):
    """Whether ra_forward runs a bf16 d_k = 128 share with a side stream as two
    chains: one to two work units (query-tile pairs x heads) per compute unit."""
    n_pairs = ((n_q + 127) // 128 + 1) // 2
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return cus <= n_pairs * h_q < 2 * cus


@pytest.mark.parametrize("n_q,n_k,n_cp", [(2000, 300, 7), (2048, 256, 2)])
def test_two_chain_schedule(n_q, n_k, n_cp):
    """A share with one to two work units per compute unit runs as two chains
    of launches (even blocks into one running state on the launch stream, odd
    blocks into another on the side stream, staging slots reused from block 5
    on) merged at the end: against the oracle like every schedule, tile counts
    exact, and within the same bound of the one-stream schedule."""
    rng = np.random.default_rng(n_q + n_cp)
    sh = _custom_share(rng, "bf16", 128, 32, 8, n_q, n_k, n_cp)
    assert _chains(32, n_q)
    check_share(sh, f"two chains nq{n_q} nk{n_k} ncp{n_cp}")
    a = run_forward(sh)
    b = run_forward(sh, side=False)
    assert np.array_equal(a[2], b[2]) and a[3] == b[3]
    compare(a[0], a[1], b[0].astype(np.float64), b[1].astype(np.float64), TOL["bf16"],
            "two chains against one stream")


def test_two_chain_edge_cases():
    """Two-chain shapes where a chain sees nothing: the odd blocks wholly
    after every query (state 1 stays empty, m = -inf, and the merge returns
    state 0's result), and blocks with no keys at all (both states empty:
    out = 0, lse = -inf)."""
    rng = np.random.default_rng(404)
    sh = _custom_share(rng, "bf16", 128, 32, 8, 2048, 256, 4)
    assert _chains(32, 2048)
    future = int(sh.q_pos.max()) + 1
    for b in (1, 3):
        sh.k_pos[b] = np.arange(future, future + 256, dtype=np.int64) + 1000 * b
    sh = sh.to_gpu()
    check_share(sh, "two chains, odd blocks in the future")
    d = 128
    q = sh.gq
    ek = torch.empty((8, 0, d), dtype=torch.bfloat16, device="cuda")
    ep = torch.empty((0,), dtype=torch.int32, device="cuda")
    out, lse, work, staged = ra.forward(q, sh.gq_pos, [ek] * 3, [ek] * 3, [ep] * 3)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    assert work.tolist() == [0, 0, 0] and staged == 0


def test_step_by_step_matches_oracle_and_forward():
    """state_init + ra_step per block + ra_finalize: after every step the
    state finalises to the oracle's, and the end result equals ra_forward
    bit for bit."""
    case = synth.case_by_name("llama405b_stage_share")
    sh = Share(case, 3, T=8192, n_cp=8).to_gpu()
    h_q, n_q, d = sh.gq.shape
    p = ra.problem(n_q, sh.gk[0].shape[1], h_q, sh.gk[0].shape[0], d, torch.bfloat16)
    m, l, o = ra.new_state(h_q, n_q, d, "cuda")
    ra.state_init(p, m, l, o)
    work = torch.zeros(3, dtype=torch.int64, device="cuda")
    st = oracle.init_state(h_q, n_q, d)
    for b in range(len(sh.gk)):
        ra.step(sh.gq, sh.gq_pos, sh.gk[b], sh.gv[b], sh.gk_pos[b], m, l, o, work)
        st = oracle.ring_step_ref(sh.q, sh.q_pos, sh.k[b], sh.v[b], sh.k_pos[b], st)
        out, lse = ra.finalize(p, m, l, o)
        ro, rl = oracle.finalize(*st)
        compare(out.cpu(), lse.cpu(), ro, rl, TOL["bf16"], f"step {b}")
        # the state itself: m is the running maximum, l the exp-sum against it
        mc, lc = m.cpu().numpy(), l.cpu().numpy()
        fin = np.isfinite(st[0])
        assert np.array_equal(np.isfinite(mc), fin)
        assert max_err(mc[fin], st[0][fin]) <= 1e-3
        assert np.abs(lc[fin] / st[1][fin] - 1).max() <= 1e-3
    fo, fl, fw, _ = run_forward(sh)
    assert np.array_equal(out.cpu().numpy(), fo) and np.array_equal(lse.cpu().numpy(), fl)
    assert np.array_equal(work.cpu().numpy(), fw)


def test_checkpoint_resume_bitwise():
    """The state after k steps, saved to the host and restored, resumes to the
    uninterrupted result bit for bit."""
    case = synth.case_by_name("million_striped_mha")
    sh = Share(case, 1, T=8192, n_cp=8).to_gpu()
    h_q, n_q, d = sh.gq.shape
    p = ra.problem(n_q, sh.gk[0].shape[1], h_q, sh.gk[0].shape[0], d, torch.bfloat16)

    def run(cut):
        m, l, o = ra.new_state(h_q, n_q, d, "cuda")
        ra.state_init(p, m, l, o)
        for b in range(len(sh.gk)):
            if b == cut:
                saved = [x.cpu() for x in (m, l, o)]
                m, l, o = [x.cuda() for x in saved]
            ra.step(sh.gq, sh.gq_pos, sh.gk[b], sh.gv[b], sh.gk_pos[b], m, l, o)
        return [x.cpu().numpy() for x in ra.finalize(p, m, l, o)]

    ref = run(-1)
    for cut in (1, 4, 7):
        got = run(cut)
        assert all(np.array_equal(a, b) for a, b in zip(ref, got))


def test_untouched_rows_and_empty_blocks():
    """A block wholly after every query leaves the state bit-identical; an
    empty block (n_k = 0) too; a share with no keys finalises to 0 / -inf."""
    rng = np.random.default_rng(13)
    sh = _custom_share(rng, "bf16", 128, 2, 1, 256, 128, 1)
    h_q, n_q, d = sh.gq.shape
    p = ra.problem(n_q, 128, h_q, 1, d, torch.bfloat16)
    m, l, o = ra.new_state(h_q, n_q, d, "cuda")
    ra.state_init(p, m, l, o)
    ra.step(sh.gq, sh.gq_pos, sh.gk[0], sh.gv[0], sh.gk_pos[0], m, l, o)
    before = [x.clone() for x in (m, l, o)]
    future = sh.gk_pos[0] + int(sh.q_pos.max()) + 1
    work = torch.zeros(3, dtype=torch.int64, device="cuda")
    ra.step(sh.gq, sh.gq_pos, sh.gk[0], sh.gv[0], future, m, l, o, work)
    for a, b in zip(before, (m, l, o)):
        assert torch.equal(a, b)
    bm, bn = ra.tile_shape(p)
    assert work.tolist() == [0, 0, (256 // bm) * (128 // bn)]  # every tile skipped
    ek = torch.empty((1, 0, d), dtype=torch.bfloat16, device="cuda")
    ep = torch.empty((0,), dtype=torch.int32, device="cuda")
    ra.step(sh.gq, sh.gq_pos, ek, ek, ep, m, l, o)
    for a, b in zip(before, (m, l, o)):
        assert torch.equal(a, b)
    out, lse, work, staged = ra.forward(sh.gq, sh.gq_pos, [ek, ek], [ek, ek], [ep, ep])
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    assert work.tolist() == [0, 0, 0] and staged == 0


def test_empty_queries():
    d = 128
    q = torch.empty((2, 0, d), dtype=torch.bfloat16, device="cuda")
    qp = torch.empty((0,), dtype=torch.int32, device="cuda")
    k = torch.randn((1, 64, d), device="cuda").to(torch.bfloat16)
    kp = torch.arange(64, dtype=torch.int32, device="cuda")
    out, lse, work, staged = ra.forward(q, qp, [k], [k], [kp])
    assert out.shape == (2, 0, d) and work.tolist() == [0, 0, 0]


def test_deterministic_and_staging_order_independent():
    """Repeat runs, runs without the side stream and runs whose side stream is
    held back by a spin kernel all give the same bits."""
    case = synth.case_by_name("llama70b_stage_share")
    sh = Share(case, 0, T=16384, n_cp=16).to_gpu()
    a = run_forward(sh)
    b = run_forward(sh)
    c = run_forward(sh, side=False)
    side = ra.side_stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)  # ~10 ms: staging starts late
    d = run_forward(sh)
    for x in (b, c, d):
        assert np.array_equal(a[0], x[0]) and np.array_equal(a[1], x[1])
        assert np.array_equal(a[2], x[2]) and a[3] == x[3]


def test_timed_forward_matches_and_reports_every_step():
    """ra_forward_timed gives ra_forward's bits, one kernel time per step and
    a staging wait that is never negative; with the side stream held back the
    copies show up as exposed wait."""
    case = synth.case_by_name("llama70b_stage_share")
    sh = Share(case, 0, T=16384, n_cp=8).to_gpu()
    f = ra.Forward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    o1, l1 = (t.clone() for t in f())
    t = f.timed()
    torch.cuda.synchronize()
    assert torch.equal(o1, f.out) and torch.equal(l1, f.lse)
    n = len(sh.gk)
    assert len(t["kernel_ms"]) == len(t["gap_ms"]) == len(t["staging_wait_ms"]) == n
    assert all(k > 0 for k in t["kernel_ms"]) and min(t["gap_ms"]) >= 0
    assert min(t["staging_wait_ms"]) >= 0 and t["total_ms"] >= sum(t["kernel_ms"])
    side = ra.side_stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)  # ~10 ms: the first copy lands late
    late = f.timed()
    assert torch.equal(o1, f.out) and torch.equal(l1, f.lse)
    assert late["staging_wait_ms"][1] > 1.0


def test_work_counts_give_pages_half_blocks():
    """Tile counters reproduce the pages' causal work: contiguous rank i does
    2i+1 half-blocks, zigzag ranks all do 4*n_cp."""
    n_cp = 4
    for layout, chunk in (("contiguous", 1024), ("zigzag", 512)):
        case = synth.Case("w", T=4096, n_cp=n_cp, layout=layout, ranks=(0,), h_q=2, h_kv=1,
                          d_k=128, dtype="bf16", seed=5)
        got = []
        for r in range(n_cp):
            sh = Share(case, r).to_gpu()
            _, _, work, _ = run_forward(sh)
            bm, bn = ra.tile_shape(ra.problem(1, 1, 2, 1, 128, torch.bfloat16))
            got.append(oracle.half_blocks_from_tiles(int(work[0]), int(work[1]), chunk, bm, bn))
        if layout == "contiguous":
            assert got == [2 * i + 1 for i in range(n_cp)]
        else:
            assert got == [4 * n_cp] * n_cp


@pytest.mark.parametrize("h_q,h_kv", [(256, 1), (256, 256), (256, 16)])
def test_max_heads(h_q, h_kv):
    """The largest head count the boundary takes (256 query heads), with one,
    every and an intermediate number of key/value heads."""
    rng = np.random.default_rng(h_kv)
    sh = _custom_share(rng, "bf16", 128, h_q, h_kv, 160, 96, 2)
    check_share(sh, f"max heads {h_q}/{h_kv}")


def test_mfma_ceiling_runs_and_reports_a_rate():
    """The matrix-pipe calibration runs on every compute unit and its rate is
    a plausible fraction of the nominal peak (the clock the chip holds under
    full matrix load is below 2.4 GHz, never above)."""
    tf, ms = ra.mfma_ceiling(iters=2048, reps=2)
    assert ms > 0 and 0.3 * 2516.6 < tf < 1.02 * 2516.6


def test_debug_check_on_device_positions(monkeypatch):
    """RA_DEBUG=1: the binding refuses positions that do not increase before
    any launch; valid positions pass through to the same results."""
    rng = np.random.default_rng(31)
    sh = _custom_share(rng, "bf16", 128, 2, 1, 130, 70, 2)
    monkeypatch.setenv("RA_DEBUG", "1")
    out, lse, _, _ = ra.forward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    ro, rl = sh.oracle()
    compare(out.cpu(), lse.cpu(), ro, rl, TOL["bf16"], "debug-checked forward")
    bad = sh.gq_pos.clone()
    bad[5] = bad[4]
    with pytest.raises(ValueError):
        ra.forward(sh.gq, bad, sh.gk, sh.gv, sh.gk_pos)


@pytest.mark.parametrize("name", ["llama405b_stage_share", "llama70b_stage_share",
                                  "llama8b_gqa_zigzag", "million_striped_mha"])
def test_split_schedule_matches_one_launch(name):
    """At full size the 405B and 8B shares run the ring as launches of two
    half grids, one on each stream, while the library's copy stream stages
    the next blocks, and launches after the first take two blocks each (the
    state kept in registers between them).  Every work unit computes exactly
    what it computes in the one-launch-per-block schedule (one stream; the
    timed call, which never splits), so the results and tile counts are the
    same bit for bit.  The 70B and striped shares (one to two work units per
    compute unit) run as two chains whose states are merged at the end: the
    same tile counts, results within the parity bound of the one-launch
    ones.  A HIP-graph replay (captured, the schedule stages on the side
    stream: split for the GQA shares, one launch per step for the striped
    one) gives the one-launch bits."""
    sh = Share(synth.case_by_name(name), 0).to_gpu()
    print(f"[parity] split schedule {name}", flush=True)
    a = run_forward(sh)              # side stream: the library's schedule
    b = run_forward(sh, side=False)  # one stream: one launch per step
    assert np.array_equal(a[2], b[2]) and a[3] == b[3]
    if _chains(sh.case.h_q, len(sh.q_pos)):
        compare(a[0], a[1], b[0].astype(np.float64), b[1].astype(np.float64), TOL["bf16"],
                f"{name}: two chains against one launch per step")
    else:
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    f = ra.Forward(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    f.timed()
    torch.cuda.synchronize()
    assert np.array_equal(f.out.cpu().numpy(), b[0]) and np.array_equal(f.lse.cpu().numpy(), b[1])
    g = ra.ForwardGraph(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    for _ in range(2):
        out, lse = g()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), b[0]) and np.array_equal(lse.cpu().numpy(), b[1])

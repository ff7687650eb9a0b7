"""Parity of the document-masked all-gather form (ra_forward_allgather_docs:
packed sequences, a key visible only within the query's document) with the
float64 oracle, which applies the mask as document ids.  Element by element
at reduced sizes on every workload, single-token and tile-aligned documents,
ragged shares on both kernels, block order, the full 405B, 70B and striped
shares on sampled rows, and one document reproducing the unmasked result
(bit for bit where no tile is split).  A query tile whose rows span more than
8192 positions from the first row's document start to the last row has its
key blocks split over several workgroups and merged; the cases marked
"split" hold such tiles, which the test checks before comparing."""

import numpy as np
import pytest
import torch

import oracle
import ring_attention_rank_amd as ra
import ring_attention_rank_amd.layouts as L
import synth
from gpu_util import TOL, Share, max_err, sample_rows
from test_gpu_parity import _custom_share, compare

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def doc_inputs(sh, starts, rows=None):
    qp = sh.q_pos if rows is None else sh.q_pos[rows]
    q_doc = oracle.doc_ids(qp, starts)
    k_doc = [oracle.doc_ids(p, starts) for p in sh.k_pos]
    lo = torch.from_numpy(L.document_start_of(sh.q_pos, starts)).cuda()
    return q_doc, k_doc, lo


def run_docs(sh, lo, order=None):
    idx = list(range(len(sh.gk))) if order is None else list(order)
    out, lse, work = ra.forward_allgather(sh.gq, sh.gq_pos, [sh.gk[i] for i in idx],
                                          [sh.gv[i] for i in idx], [sh.gk_pos[i] for i in idx],
                                          q_doc_start=lo)
    torch.cuda.synchronize()
    assert work is None
    return out.cpu().numpy(), lse.cpu().numpy()




def split_tiles(sh, starts):
    """Query tiles (128 rows) of the share whose key walk is split."""
    lo = L.document_start_of(sh.q_pos, starts)
    n = sh.q_pos.size
    return sum(int(sh.q_pos[min(t + 128, n) - 1] - lo[t] > ra.docs_split_span()) for t in range(0, n, 128))


def check_docs(sh, starts, label):
    print(f"[docs] {label}: {len(starts)} documents, {split_tiles(sh, starts)} split tiles",
          flush=True)
    q_doc, k_doc, lo = doc_inputs(sh, starts)
    out, lse = run_docs(sh, lo)
    ro, rl = oracle.ring_forward_ref(sh.q, sh.q_pos, sh.k, sh.v, sh.k_pos,
                                     q_doc=q_doc, k_doc_blocks=k_doc)
    return compare(out, lse, ro, rl, TOL[sh.case.dtype], label)


@pytest.mark.parametrize("name,T,n_cp,rank,lens", [
    ("tiny_f32_contiguous", 1024, 4, 2, (16, 400)),
    ("llama8b_gqa_zigzag", 4096, 4, 1, (64, 2048)),
    ("llama70b_stage_share", 8192, 16, 15, (64, 4096)),
    ("llama405b_stage_share", 8192, 16, 0, (64, 4096)),
    ("million_striped_mha", 16384, 64, 5, (128, 4096)),
])
def test_reduced_configs(name, T, n_cp, rank, lens):
    case = synth.case_by_name(name)
    sh = Share(case, rank, T=T, n_cp=n_cp).to_gpu()
    starts = synth.document_starts(T, case.seed, *lens)
    check_docs(sh, starts, f"{name}@T{T}/r{rank}")


@pytest.mark.parametrize("name,T,n_cp,rank,lens", [
    ("llama70b_stage_share", 32768, 16, 15, (4096, 32768)),   # every tile split
    ("llama405b_stage_share", 32768, 16, 0, (2048, 16384)),   # half of them
    ("million_striped_mha", 65536, 64, 5, (128, 4096)),       # 6 of 8, 8 KV heads
])
def test_split_tiles(name, T, n_cp, rank, lens):
    """Long documents, so that late rows see keys of many blocks: those
    tiles are split over workgroups and their partial states merged, next
    to tiles folded whole in the same launch."""
    case = synth.case_by_name(name)
    sh = Share(case, rank, T=T, n_cp=n_cp).to_gpu()
    starts = synth.document_starts(T, case.seed, *lens)
    n_split = split_tiles(sh, starts)
    assert n_split > 0
    check_docs(sh, starts, f"{name}@T{T}/r{rank} split")


@pytest.mark.parametrize("seed", [31, 32])
def test_split_tiles_ragged(seed):
    """Ragged sizes with split tiles: 517 queries (a last tile of 5 rows,
    split with seed 31, whole with seed 32), 1100 keys a block over 6 blocks
    (a ragged last key tile), random sparse positions and four documents."""
    rng = np.random.default_rng(seed)
    sh = _custom_share(rng, "bf16", 128, 4, 1, 517, 1100, 6)
    span = int(max(sh.q_pos.max(), max(p.max() for p in sh.k_pos))) + 1
    starts = np.concatenate([[0], np.sort(rng.choice(np.arange(1, span), 3, replace=False))])
    assert 0 < split_tiles(sh, starts) < 5
    check_docs(sh, starts, f"ragged split seed {seed}")


@pytest.mark.parametrize("name", ["llama405b_stage_share", "tiny_f32_contiguous"])
def test_single_token_and_aligned_documents(name):
    """Documents of one token, documents that start on wave (32), tile (64)
    and workgroup (128) boundaries, and one that starts a token past one."""
    case = synth.case_by_name(name)
    T, n_cp = (8192, 16) if case.dtype == "bf16" else (1024, 4)
    sh = Share(case, n_cp - 1, T=T, n_cp=n_cp).to_gpu()
    starts = np.array(sorted({0, 5, 6, 7, 32, 64, 65, 128, 129, 300, 301, 302, 512, T // 2,
                              T // 2 + 1, T - 64, T - 3, T - 2, T - 1}))
    check_docs(sh, starts, f"{name} single-token and aligned documents")


@pytest.mark.parametrize("name,T,n_cp", [("llama405b_stage_share", 32768, 16),
                                          ("llama405b_stage_share", 8192, 16),
                                          ("llama8b_gqa_zigzag", 8192, 1),
                                          ("tiny_f32_contiguous", 1024, 4)])
def test_one_document_is_the_unmasked_result(name, T, n_cp):
    """Split tiles (the 405B share at T = 32768: its late chunk's tiles span
    more than 8192 positions) merge partial states in another order than the
    one-launch fold, so agree to rounding.  So does a plain launch of at least
    two tile pairs x heads per compute unit, which folds each tile's keys in
    one group where the document-masked launch folds two interleaved halves
    and merges them.  Otherwise (shorter spans, a single block, the fp32 path)
    the result is the same bit for bit."""
    case = synth.case_by_name(name)
    sh = Share(case, 0, T=T, n_cp=n_cp).to_gpu()
    _, _, lo = doc_inputs(sh, np.array([0]))
    out, lse = run_docs(sh, lo)
    ref_out, ref_lse, _ = ra.forward_allgather(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos)
    torch.cuda.synchronize()
    ref_out, ref_lse = ref_out.cpu().numpy(), ref_lse.cpu().numpy()
    h_q, n_q = sh.gq.shape[0], sh.gq.shape[1]
    one_group = (case.dtype == "bf16" and case.d_k == 128 and
                 ((n_q + 127) // 128 + 1) // 2 * h_q >=
                 2 * torch.cuda.get_device_properties(0).multi_processor_count)
    if case.dtype == "bf16" and (n_cp > 1 and split_tiles(sh, np.array([0])) > 0 or one_group):
        tol = TOL["bf16"]
        assert max_err(out, ref_out) <= tol["out"] and max_err(lse, ref_lse) <= tol["lse"]
    else:
        assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)


@pytest.mark.parametrize("dtype,d_k", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_ragged_random_documents(dtype, d_k):
    rng = np.random.default_rng(21 + d_k)
    sh = _custom_share(rng, dtype, d_k, 4, 2, 517, 129, 3)
    span = int(max(sh.q_pos.max(), max(p.max() for p in sh.k_pos))) + 1
    starts = np.concatenate([[0], np.sort(rng.choice(np.arange(1, span), 40, replace=False))])
    check_docs(sh, starts, f"ragged {dtype} d{d_k}")


def test_block_order_does_not_matter():
    case = synth.case_by_name("llama8b_gqa_zigzag")
    sh = Share(case, 2, T=4096, n_cp=4).to_gpu()
    _, _, lo = doc_inputs(sh, synth.document_starts(4096, case.seed, 64, 2048))
    a_out, a_lse = run_docs(sh, lo)
    b_out, b_lse = run_docs(sh, lo, order=[3, 1, 0, 2])
    tol = TOL["bf16"]
    assert max_err(a_out, b_out) <= tol["out"] and max_err(a_lse, b_lse) <= tol["lse"]


@pytest.mark.parametrize("name", ["llama405b_stage_share", "llama70b_stage_share",
                                  "million_striped_mha"])
def test_full_size_sampled(name):
    """Full stage shares (T = 131072 over 16 zigzag blocks; the striped one
    T = 524288 over 64 blocks) with the sequence packed from documents of 512
    to 32768 tokens."""
    case = synth.case_by_name(name)
    sh = Share(case, case.ranks[0]).to_gpu()
    starts = synth.document_starts(case.T, case.seed)
    print(f"[docs] {name} full size, {len(starts)} documents", flush=True)
    _, _, lo = doc_inputs(sh, starts)
    out, lse, _ = ra.forward_allgather(sh.gq, sh.gq_pos, sh.gk, sh.gv, sh.gk_pos, q_doc_start=lo)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    rows = sample_rows(sh.q_pos, seed=9)
    # also the first rows of documents inside the share, where windows are short
    firsts = np.searchsorted(sh.q_pos, starts)
    rows = np.unique(np.concatenate([rows, firsts[firsts < sh.q_pos.size]]))
    q_doc, k_doc, _ = doc_inputs(sh, starts, rows)
    ro, rl = oracle.ring_forward_ref(sh.q[:, rows], sh.q_pos[rows], sh.k, sh.v, sh.k_pos,
                                     q_doc=q_doc, k_doc_blocks=k_doc)
    idx = torch.from_numpy(rows).cuda()
    eo = max_err(out[:, idx].cpu().numpy(), ro)
    el = max_err(lse[:, idx].cpu().numpy(), rl)
    print(f"[docs] {name}: out err {eo:.3e} lse err {el:.3e}", flush=True)
    assert eo <= TOL["bf16"]["out"] and el <= TOL["bf16"]["lse"]


@pytest.mark.parametrize("name,T", [("llama8b_gqa_zigzag", 8192), ("tiny_f32_contiguous", 1024)])
def test_single_block_packed_sequence(name, T):
    """One rank holding the whole sequence (n_cp = 1, as in the Ulysses share):
    plain causal attention over a packed sequence, one resident block."""
    case = synth.case_by_name(name)
    sh = Share(case, 0, T=T, n_cp=1).to_gpu()
    starts = synth.document_starts(T, case.seed + 7, 16, T // 4)
    check_docs(sh, starts, f"{name}@T{T} single block")


def test_empty_queries_and_blocks():
    """No queries: nothing to do.  Blocks without keys: every query's document
    has no key, so out = 0 and lse = -inf (the entry point's stated result)."""
    d = 128
    q = torch.empty((2, 0, d), dtype=torch.bfloat16, device="cuda")
    qp = torch.empty((0,), dtype=torch.int32, device="cuda")
    k = torch.randn((1, 64, d), device="cuda").to(torch.bfloat16)
    kp = torch.arange(64, dtype=torch.int32, device="cuda")
    out, lse, _ = ra.forward_allgather(q, qp, [k, k], [k, k], [kp, kp + 64], q_doc_start=qp)
    assert out.shape == (2, 0, d) and lse.shape == (2, 0)
    q = torch.randn((2, 200, d), device="cuda").to(torch.bfloat16)
    qp = torch.arange(200, dtype=torch.int32, device="cuda")
    k0 = torch.empty((1, 0, d), dtype=torch.bfloat16, device="cuda")
    kp0 = torch.empty((0,), dtype=torch.int32, device="cuda")
    out, lse, _ = ra.forward_allgather(q, qp, [k0, k0], [k0, k0], [kp0, kp0],
                                       q_doc_start=torch.zeros_like(qp))
    torch.cuda.synchronize()
    assert bool((out == 0).all()) and bool(torch.isneginf(lse).all())


@pytest.mark.parametrize("h_kv", [1, 256])
def test_max_heads_split(h_kv):
    """The largest head count the boundary takes (256 query heads) with split
    tiles: positions spread 64 apart so that a 128-row tile spans well over
    8192 positions, two documents."""
    rng = np.random.default_rng(40 + h_kv)
    sh = _custom_share(rng, "bf16", 128, 256, h_kv, 160, 96, 2)
    sh.q_pos = sh.q_pos * 64
    sh.k_pos = [p * 64 for p in sh.k_pos]
    sh.to_gpu()
    span = int(max(sh.q_pos.max(), max(p.max() for p in sh.k_pos))) + 1
    starts = np.array([0, span // 3])
    assert split_tiles(sh, starts) > 0
    check_docs(sh, starts, f"max heads 256/{h_kv} split")

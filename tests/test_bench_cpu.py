"""bench.py's host logic, without a GPU: the single-GPU guard and the rule
that the committed HBM traffic figure is reported only for its own workload
and while the kernel source still has the hash it was measured at."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _summary(tmp_path, workload, sha, value="1.6e8"):
    f = tmp_path / "traffic.md"
    f.write_text(f"# traffic\n\n- workload: {workload}\n- kernel_source_sha256: {sha}\n"
                 f"- hbm_bytes_per_launch: {value}\n")
    return str(f)


def test_traffic_figure_matches_its_workload_only(monkeypatch, tmp_path):
    sha = bench.kernel_source_sha256()
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", _summary(tmp_path, "llama405b_stage_share", sha))
    assert bench.committed_traffic("llama405b_stage_share") == 1.6e8
    assert bench.committed_traffic("llama70b_stage_share") is None


def test_traffic_figure_dropped_when_the_kernel_changes(monkeypatch, tmp_path):
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY",
                        _summary(tmp_path, "llama405b_stage_share", bench.kernel_source_sha256()))
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "0" * 64)
    assert bench.committed_traffic("llama405b_stage_share") is None


def test_traffic_figure_missing_summary(monkeypatch, tmp_path):
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "absent.md"))
    assert bench.committed_traffic("llama405b_stage_share") is None


def test_document_mask_pair_count_matches_brute_force():
    import numpy as np
    import oracle
    import ring_attention_rank_amd as ra
    starts = np.array([0, 17, 40, 41, 100, 200])
    for layout in ("contiguous", "zigzag", "striped"):
        qp = oracle.positions(256, 4, 1, layout)
        for s in range(4):
            kp = oracle.positions(256, 4, s, layout)
            lo = ra.layouts.document_start_of(qp, starts)
            same = oracle.doc_ids(kp, starts)[None, :] == oracle.doc_ids(qp, starts)[:, None]
            brute = int(((kp[None, :] <= qp[:, None]) & same).sum())
            assert bench.visible_pairs_docs(qp, lo, kp) == brute


def test_comm_model_of_the_405b_share():
    """The pages' exchange model for the headline share: 15 incoming blocks of
    4 MiB (the 63 MB of the pages), Ulysses' break-even group 1 + 16/1, and
    the link rate that lands one block within one step."""
    case = synth.case_by_name("llama405b_stage_share")
    m = bench.comm_model(case, 62914560, 0.25)
    assert m["ring_bytes_per_layer"] == m["staged_bytes_measured"] == 15 * 4194304
    assert m["kv_block_bytes"] == 4194304 and m["ulysses_breakeven_group"] == 17
    assert m["ulysses_bytes_per_layer"] > m["ring_bytes_per_layer"]  # n_cp = 16 < 17
    assert abs(m["link_GBps_to_hide_each_step"] - 4194304 / 0.25e-3 / 1e9) < 1e-9

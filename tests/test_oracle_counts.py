"""Work, tile and byte counts of the oracle against the pages' figures,
closed forms and brute-force counting."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def test_contiguous_work_matches_pages():
    assert oracle.causal_work(oracle.chunk_assignment(4, "contiguous")) == \
        GOLD["contiguous_blocks_per_gpu_n4"]["value"]
    for n in range(1, 33):
        w = oracle.causal_work(oracle.chunk_assignment(n, "contiguous"))
        assert w[-1] / w[0] == 2 * n - 1  # last GPU / first GPU
        assert w == [i + 0.5 for i in range(n)]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16, 64])
def test_zigzag_work_is_equal(n):
    assert GOLD["zigzag_equal"]["value"]
    w = oracle.causal_work(oracle.chunk_assignment(n, "zigzag"))
    assert len(set(w)) == 1
    # 2n chunk-pair blocks per GPU: chunk i gives i + 1/2, its mirror 2n-1-i + 1/2
    assert w[0] == 2 * n
    # and the whole triangle is covered: (2n)^2 / 2
    assert sum(w) == (2 * n) ** 2 / 2


def _brute_pairs(qp, kp):
    return int((np.asarray(kp)[None, :] <= np.asarray(qp)[:, None]).sum())


@pytest.mark.parametrize("layout", oracle.LAYOUTS)
def test_visible_pairs_closed_forms(layout):
    for T, n_cp in [(64, 4), (96, 4), (256, 8)]:
        n = T // n_cp
        c = T // (2 * n_cp)
        total = 0
        for r in range(n_cp):
            qp = oracle.positions(T, n_cp, r, layout)
            pr = 0
            for s in oracle.ring_sources(n_cp, r):
                kp = oracle.positions(T, n_cp, s, layout)
                got = oracle.visible_pairs(qp, kp)
                assert got == _brute_pairs(qp, kp)
                pr += got
            if layout == "contiguous":
                assert pr == r * n * n + n * (n + 1) // 2
            elif layout == "zigzag":
                assert pr == 2 * n_cp * c * c + c
            else:
                assert pr == n_cp * n * (n - 1) // 2 + (r + 1) * n
            total += pr
        assert total == T * (T + 1) // 2


def test_visible_pairs_noncausal():
    assert oracle.visible_pairs(np.arange(5), np.arange(100, 107), causal=False) == 35


def _brute_tiles(qp, kp, BM, BN):
    full = masked = skipped = 0
    for i0 in range(0, len(qp), BM):
        for j0 in range(0, len(kp), BN):
            cls = set()
            for i in range(i0, min(i0 + BM, len(qp))):
                for j in range(j0, min(j0 + BN, len(kp))):
                    cls.add(bool(kp[j] <= qp[i]))
            if cls == {True}:
                full += 1
            elif cls == {False}:
                skipped += 1
            else:
                masked += 1
    return full, masked, skipped


def test_tile_work_brute_small_and_ragged():
    rng = np.random.default_rng(0)
    for _ in range(20):
        qp = np.sort(rng.choice(200, size=rng.integers(1, 40), replace=False))
        kp = np.sort(rng.choice(200, size=rng.integers(1, 40), replace=False))
        BM, BN = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        assert oracle.tile_work(qp, kp, BM, BN) == _brute_tiles(qp, kp, BM, BN)
    # one-by-one tiles count pairs
    qp, kp = np.arange(0, 30, 3), np.arange(0, 30, 2)
    f, m, s = oracle.tile_work(qp, kp, 1, 1)
    assert m == 0 and f == oracle.visible_pairs(qp, kp) and f + s == qp.size * kp.size
    assert oracle.tile_work(qp, kp, 4, 4, causal=False) == (3 * 4, 0, 0)


@pytest.mark.parametrize("n_cp", [2, 4, 8])
def test_half_blocks_from_tiles_match_pages(n_cp):
    # contiguous: GPU i does 2i+1 half-blocks; zigzag: 4 n_cp each
    T = 64 * 2 * n_cp
    for layout, chunk in (("contiguous", T // n_cp), ("zigzag", T // (2 * n_cp))):
        BM = BN = 16
        per_rank = []
        for r in range(n_cp):
            qp = oracle.positions(T, n_cp, r, layout)
            f = m = 0
            for s in oracle.ring_sources(n_cp, r):
                ff, mm, _ = oracle.tile_work(qp, oracle.positions(T, n_cp, s, layout), BM, BN)
                f, m = f + ff, m + mm
            per_rank.append(oracle.half_blocks_from_tiles(f, m, chunk, BM, BN))
        if layout == "contiguous":
            assert per_rank == [2 * i + 1 for i in range(n_cp)]
        else:
            assert per_rank == [4 * n_cp] * n_cp


def test_striped_tiles_per_block():
    # with square tiles every (r, s) block has (n/b)(n/b-1)/2 full tiles and n/b masked
    T, n_cp, b = 512, 4, 8
    n = T // n_cp
    for r in range(n_cp):
        qp = oracle.positions(T, n_cp, r, "striped")
        for s in range(n_cp):
            f, m, sk = oracle.tile_work(qp, oracle.positions(T, n_cp, s, "striped"), b, b)
            assert (f, m) == ((n // b) * (n // b - 1) // 2, n // b)
            assert f + m + sk == (n // b) ** 2


def test_llama405b_allgather_bytes():
    g = GOLD["llama405b_stage"]
    d_kv = g["kv_heads_per_gpu"] * g["d_k"]
    assert g["q_heads"] // g["t"] == 16 and g["kv_heads"] // g["t"] == g["kv_heads_per_gpu"]
    assert g["T"] // g["n_cp"] == g["queries_per_gpu"]
    ring = oracle.cp_comm_bytes(g["T"], g["d"] // g["t"], d_kv, g["n_cp"], "ring")
    ag = oracle.cp_comm_bytes(g["T"], g["d"] // g["t"], d_kv, g["n_cp"], "allgather")
    assert ring == ag == 62_914_560
    assert round(ring / 1e6) == g["allgather_MB_per_gpu_per_layer"]
    # the exercise stub's placeholder 4*T*d_kv would be 67 MB, not 63
    assert round(4 * g["T"] * d_kv / 1e6) != g["allgather_MB_per_gpu_per_layer"]
    # without GQA each GPU holds as many KV heads as query heads: 16x the bytes
    no_gqa = oracle.cp_comm_bytes(g["T"], g["d"] // g["t"], 16 * g["d_k"], g["n_cp"], "ring")
    assert no_gqa == g["no_gqa_multiplier"] * ring
    # per block: 4 n d_kv bytes in 16 bits
    assert oracle.kv_block_bytes(8192, d_kv) == 4 * 8192 * d_kv == 4_194_304


def test_ulysses_breakeven_and_byte_model():
    g = GOLD["ulysses_breakeven"]
    assert oracle.ulysses_breakeven(8, 8) == g["no_gqa"]
    assert oracle.ulysses_breakeven(64, 8) == g["gqa_8_to_1"]
    # Ulysses needs whole KV heads per GPU: at most n_kv = 8 GPUs, short of 9
    assert 8 == g["llama_ulysses_max_gpus"] < g["gqa_8_to_1"]
    # the break-even agrees with the two byte models it comes from
    d_k = 128
    for h, n_kv in [(8, 8), (64, 8), (32, 8), (16, 1), (12, 4)]:
        be = oracle.ulysses_breakeven(h, n_kv)
        for n_cp in range(2, 40):
            T = n_cp * 1024
            ring = oracle.cp_comm_bytes(T, h * d_k, n_kv * d_k, n_cp, "ring")
            uly = oracle.cp_comm_bytes(T, h * d_k, n_kv * d_k, n_cp, "ulysses")
            assert (uly < ring) == (n_cp > be), (h, n_kv, n_cp)
            assert (uly == ring) == (n_cp == be)


def test_overlap_threshold_and_flops():
    f = GOLD["gqa_overlap_factor_llama"]["value"]
    base = oracle.overlap_min_tokens(1e15, 1e11, 8, 8)
    assert abs(oracle.overlap_min_tokens(1e15, 1e11, 64, 8) * f - base) < 1e-6
    assert 131072 // 16 == GOLD["tokens_per_gpu_128k_over_16"]["value"]
    # a fully visible n x n block of h heads costs 4 n^2 d with d = h d_k
    n, h, d_k = 256, 4, 64
    pairs = oracle.visible_pairs(np.arange(n) + n, np.arange(n))
    assert pairs == n * n
    assert oracle.visible_flops(pairs, d_k, h) == 4 * n * n * (h * d_k)
    # and the send hides exactly at the bound
    F, B, n_kv = 2.0e15, 1.5e11, 1
    nmin = oracle.overlap_min_tokens(F, B, h, n_kv)
    t_comp = 4 * nmin ** 2 * (h * d_k) / F
    t_comm = 4 * nmin * (n_kv * d_k) / B
    assert abs(t_comp - t_comm) / t_comm < 1e-12


def test_bad_arguments():
    with pytest.raises(ValueError):
        oracle.chunk_assignment(4, "striped")
    with pytest.raises(ValueError):
        oracle.cp_comm_bytes(100, 8, 8, 3, "ring")
    with pytest.raises(ValueError):
        oracle.cp_comm_bytes(96, 8, 8, 3, "broadcast")

"""The package's byte model against the oracle's (each pinned separately:
the oracle's to the pages' printed figures in test_oracle_counts.py) and the
pages' own figures."""

import itertools
import math

import oracle
from ring_attention_rank_amd import comm


def test_matches_oracle():
    for T, n_cp, d, d_kv, eb in itertools.product((8192, 131072), (2, 4, 16), (1024, 16384),
                                                 (128, 1024), (2, 4)):
        for method in ("ring", "allgather", "ulysses"):
            a = comm.cp_comm_bytes(T, d, d_kv, n_cp, method, eb)
            b = oracle.cp_comm_bytes(T, d, d_kv, n_cp, method, eb)
            assert math.isclose(a, b, rel_tol=1e-12), (T, n_cp, d, d_kv, eb, method)
    for h, n_kv in ((64, 8), (128, 8), (16, 16)):
        assert comm.ulysses_breakeven(h, n_kv) == oracle.ulysses_breakeven(h, n_kv)
    assert math.isclose(comm.overlap_min_tokens(989e12, 450e9, 64, 8),
                        oracle.overlap_min_tokens(989e12, 450e9, 64, 8))


def test_pages_figures():
    # Llama-3-405B long-context stage, one key/value head per GPU after TP=8:
    # 15 blocks of 8192 tokens x 128 x 2 (K and V) x 2 bytes = "63 MB"
    assert comm.cp_comm_bytes(131072, 16 * 128, 128, 16, "allgather") == 62_914_560
    # without GQA, 16 times as much
    assert comm.cp_comm_bytes(131072, 16 * 128, 16 * 128, 16, "ring") == 16 * 62_914_560
    # Ulysses breaks even at 2 GPUs without GQA and 9 with 8 query heads per KV head
    assert comm.ulysses_breakeven(8, 8) == 2 and comm.ulysses_breakeven(64, 8) == 9

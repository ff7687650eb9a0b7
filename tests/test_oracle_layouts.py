"""Layouts, ring order and chunk assignment of the oracle."""

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("layout", oracle.LAYOUTS)
@pytest.mark.parametrize("T,n_cp", [(16, 2), (64, 4), (96, 3), (4096, 16)])
def test_positions_partition_the_sequence(layout, T, n_cp):
    seen = np.concatenate([oracle.positions(T, n_cp, r, layout) for r in range(n_cp)])
    assert np.array_equal(np.sort(seen), np.arange(T))
    for r in range(n_cp):
        p = oracle.positions(T, n_cp, r, layout)
        assert p.size == T // n_cp
        assert np.all(np.diff(p) > 0), "local positions must increase"


@pytest.mark.parametrize("T,n_cp", [(16, 2), (64, 4), (128, 8)])
def test_positions_agree_with_chunk_assignment(T, n_cp):
    # contiguous: chunk r of n_cp chunks; zigzag: chunks r, 2n_cp-1-r of 2n_cp
    for layout, n_chunks in (("contiguous", n_cp), ("zigzag", 2 * n_cp)):
        size = T // n_chunks
        for r, chunks in enumerate(oracle.chunk_assignment(n_cp, layout)):
            expect = np.concatenate([np.arange(c * size, (c + 1) * size) for c in chunks])
            assert np.array_equal(oracle.positions(T, n_cp, r, layout), expect)
    for r, toks in enumerate(oracle.chunk_assignment(n_cp, "striped", n_chunks=T)):
        assert np.array_equal(oracle.positions(T, n_cp, r, "striped"), np.array(toks))
        assert all(t % n_cp == r for t in toks)


def test_zigzag_rank0_holds_first_and_last_chunk():
    # rank 0 of a zigzag split gets the first chunk and the last
    p = oracle.positions(131072, 16, 0, "zigzag")
    assert p[0] == 0 and p[4095] == 4095 and p[4096] == 131072 - 4096 and p[-1] == 131071


def test_ring_sources():
    for n_cp in (1, 2, 5, 16):
        for r in range(n_cp):
            src = oracle.ring_sources(n_cp, r)
            assert src[0] == r
            assert sorted(src) == list(range(n_cp))
            # each step the block moves one rank to the right
            for b in range(1, n_cp):
                assert (src[b] + b) % n_cp == r


def test_bad_arguments():
    with pytest.raises(ValueError):
        oracle.positions(10, 4, 0, "contiguous")
    with pytest.raises(ValueError):
        oracle.positions(12, 4, 0, "zigzag")
    with pytest.raises(ValueError):
        oracle.positions(16, 4, 4, "striped")
    with pytest.raises(ValueError):
        oracle.positions(16, 4, 0, "diagonal")

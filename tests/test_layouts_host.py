"""The package's host-side layout helper agrees with the oracle's."""

import numpy as np
import pytest

import oracle
from ring_attention_rank_amd import layouts


@pytest.mark.parametrize("layout", oracle.LAYOUTS)
def test_positions_agree(layout):
    for T, n_cp in [(64, 4), (1024, 4), (32768, 4), (131072, 16), (524288, 64)]:
        for r in sorted({0, 1, n_cp - 1}):
            a = layouts.rank_positions(T, n_cp, r, layout)
            assert a.dtype == np.int32
            assert np.array_equal(a, oracle.positions(T, n_cp, r, layout))


def test_ring_owner_agrees():
    for n_cp in (1, 4, 16):
        for r in range(n_cp):
            assert [layouts.ring_block_owner(n_cp, r, b) for b in range(n_cp)] == oracle.ring_sources(n_cp, r)

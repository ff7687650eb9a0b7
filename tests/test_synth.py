"""The seeded input generator: deterministic, layout-independent, bf16-exact."""

import numpy as np
import torch

import synth


def test_rows_are_deterministic_and_position_indexed():
    pos = np.array([5, 4095, 4096, 9000, 3])
    a = synth.global_rows(7, synth.TENSOR_K, 2, 16, pos)
    b = synth.global_rows(7, synth.TENSOR_K, 2, 16, pos[::-1].copy())
    assert np.array_equal(a, b[:, ::-1])
    full = synth.global_rows(7, synth.TENSOR_K, 2, 16, np.arange(9100))
    assert np.array_equal(full[:, pos], a)
    c = synth.global_rows(7, synth.TENSOR_V, 2, 16, pos)
    assert not np.array_equal(a, c)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 3).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0]  # ties to even either way
    r = synth.round_to_bf16(x)
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(r, t)
    assert np.array_equal(synth.bf16_bits(r), torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_amplitude_and_dtype():
    pos = np.arange(64)
    a1 = synth.global_rows(9, 0, 1, 8, pos, amp=1.0, bf16=False)
    a2 = synth.global_rows(9, 0, 1, 8, pos, amp=2.0, bf16=False)
    assert np.array_equal(a2, 2 * a1)
    b = synth.global_rows(9, 0, 1, 8, pos, amp=1.0, bf16=True)
    assert np.array_equal(b, synth.round_to_bf16(a1))


def test_cases():
    names = [c.name for c in synth.CASES]
    assert len(names) == 5 and len(set(names)) == 5
    for c in synth.CASES:
        assert c.T % c.n_cp == 0 and c.h_q % c.h_kv == 0
    c4 = synth.case_by_name("llama405b_stage_share")
    assert (c4.T, c4.n_cp, c4.h_q, c4.h_kv, c4.d_k, c4.n) == (131072, 16, 16, 1, 128, 8192)

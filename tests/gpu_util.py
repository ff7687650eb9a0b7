"""Shared helpers of the GPU parity tests: build a rank share from the seeded
generator, move it to the GPU, and run the oracle on the same values."""

import numpy as np
import torch

import oracle
import synth

TOL = {"bf16": dict(out=1e-2, lse=1e-3), "f32": dict(out=1e-4, lse=1e-4)}


def torch_dtype(case):
    return torch.bfloat16 if case.dtype == "bf16" else torch.float32


class Share:
    """One rank's share: host inputs (float32 values of the case dtype) and
    their GPU copies, blocks in ring order."""

    def __init__(self, case, rank, T=None, n_cp=None):
        if T is not None:
            case = case.reduced(T, n_cp=n_cp)
        self.case = case
        self.rank = rank
        n_cp = case.n_cp
        self.q_pos = oracle.positions(case.T, n_cp, rank, case.layout)
        self.sources = oracle.ring_sources(n_cp, rank)
        self.k_pos = [oracle.positions(case.T, n_cp, s, case.layout) for s in self.sources]
        self.q, self.k, self.v = synth.case_inputs(case, self.q_pos, self.k_pos)

    def to_gpu(self, device="cuda"):
        dt = torch_dtype(self.case)
        self.gq = torch.from_numpy(self.q).to(dt).to(device).contiguous()
        self.gq_pos = torch.from_numpy(self.q_pos.astype(np.int32)).to(device)
        n_cp = len(self.k)
        h_kv, n_k, d = self.k[0].shape
        kk = torch.empty((n_cp, h_kv, n_k, d), dtype=dt, device=device)
        vv = torch.empty((n_cp, h_kv, n_k, d), dtype=dt, device=device)
        for b in range(n_cp):
            kk[b].copy_(torch.from_numpy(self.k[b]).to(dt))
            vv[b].copy_(torch.from_numpy(self.v[b]).to(dt))
        self.gk = [kk[b] for b in range(n_cp)]
        self.gv = [vv[b] for b in range(n_cp)]
        self.gk_pos = [torch.from_numpy(p.astype(np.int32)).to(device) for p in self.k_pos]
        return self

    def oracle(self, rows=None):
        """Oracle (out, lse) for all rows or the given local row indices."""
        q, qp = self.q, self.q_pos
        if rows is not None:
            q, qp = q[:, rows], qp[rows]
        return oracle.ring_forward_ref(q, qp, self.k, self.v, self.k_pos, causal=self.case.causal)

    def tile_work(self, BM, BN):
        tot = np.zeros(3, dtype=np.int64)
        for kp in self.k_pos:
            tot += np.array(oracle.tile_work(self.q_pos, kp, BM, BN, self.case.causal))
        return tot

    def staged_bytes(self):
        h_kv, n_k, d = self.k[0].shape
        el = 2 if self.case.dtype == "bf16" else 4
        return (len(self.k) - 1) * 2 * h_kv * n_k * d * el


def max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.abs(a - b).max())


def sample_rows(q_pos, n_rand=40, seed=0):
    """Local row indices to check at full size: both ends, every 4096-token
    chunk boundary, tile boundaries and random rows."""
    n = len(q_pos)
    rng = np.random.default_rng(seed)
    rows = {0, 1, 63, 64, 255, 256, n - 1, n - 2, n - 64, n - 65}
    for i in range(1, n):
        if q_pos[i] - q_pos[i - 1] > 1 and len(rows) < 40:
            rows.update({i - 1, i})
    rows.update(int(x) for x in rng.integers(0, n, n_rand))
    return np.array(sorted(r for r in rows if 0 <= r < n))

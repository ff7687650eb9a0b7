"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no attention arithmetic.  It defines, for every workload,
a global tensor X[tensor][head][token][d_k] of seeded random values and hands
out the rows at whatever global token positions the caller asks for, so any
layout (contiguous, zigzag, striped) slices the same global sequence.  The
caller computes the positions itself.

Recipe: values are drawn per 4096-token global chunk.  Chunk c of tensor t
(0 = Q, 1 = K, 2 = V, 3 = the output gradient dO of the backward) of a workload with seed S is
``numpy.random.Generator(PCG64(SeedSequence([S, t, c]))).standard_normal(
(heads, 4096, d_k), float32)``, multiplied by the tensor's amplitude (1 or 2,
both exact), and for 16-bit workloads rounded once to bfloat16 with
round-to-nearest-even.  The float32 arrays returned hold exactly the values
both sides use.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import CASES, ULYSSES_CASES, Case, case_by_name  # noqa: F401

CHUNK = 4096
TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DOUT = 0, 1, 2, 3
_THREADS = 8


def round_to_bf16(x):
    """Round float32 values to the nearest bfloat16 value (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    Inputs here are finite normals, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def bf16_bits(x):
    """Upper 16 bits of bfloat16-representable float32 values (uint16)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _chunk(seed, tensor_id, chunk_id, n_heads, d_k, amp, bf16):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, chunk_id])))
    x = rng.standard_normal((n_heads, CHUNK, d_k), dtype=np.float32)
    if amp != 1.0:
        x *= np.float32(amp)
    if bf16:
        x = round_to_bf16(x)
    return x


def global_rows(seed, tensor_id, n_heads, d_k, pos, amp=1.0, bf16=True):
    """Rows of global tensor ``tensor_id`` at global positions ``pos``.

    Returns float32 ``[n_heads][len(pos)][d_k]``.
    """
    pos = np.asarray(pos, dtype=np.int64)
    out = np.empty((n_heads, pos.size, d_k), dtype=np.float32)
    if pos.size == 0:
        return out
    chunks = np.unique(pos // CHUNK)

    def work(c):
        x = _chunk(seed, tensor_id, int(c), n_heads, d_k, amp, bf16)
        sel = np.nonzero(pos // CHUNK == c)[0]
        out[:, sel, :] = x[:, pos[sel] - c * CHUNK, :]

    if chunks.size == 1:
        work(chunks[0])
    else:
        with ThreadPoolExecutor(min(_THREADS, chunks.size)) as ex:
            list(ex.map(work, chunks))
    return out


def case_inputs(case, q_pos, k_pos_blocks):
    """Q rows at ``q_pos`` and K, V rows for every block's positions.

    Returns (q, k_blocks, v_blocks) as float32 arrays holding the exact values
    of the workload's dtype.
    """
    bf16 = case.dtype == "bf16"
    q = global_rows(case.seed, TENSOR_Q, case.h_q, case.d_k, q_pos, case.q_amp, bf16)
    allk = np.concatenate([np.asarray(p, dtype=np.int64) for p in k_pos_blocks]) if k_pos_blocks else np.zeros(0, np.int64)
    kk = global_rows(case.seed, TENSOR_K, case.h_kv, case.d_k, allk, case.k_amp, bf16)
    vv = global_rows(case.seed, TENSOR_V, case.h_kv, case.d_k, allk, case.v_amp, bf16)
    k_blocks, v_blocks = [], []
    o = 0
    for p in k_pos_blocks:
        n = len(p)
        k_blocks.append(np.ascontiguousarray(kk[:, o:o + n]))
        v_blocks.append(np.ascontiguousarray(vv[:, o:o + n]))
        o += n
    return q, k_blocks, v_blocks


def case_dout(case, q_pos):
    """Output gradient rows (amplitude 1) at the local query positions,
    ``[h_q][len(q_pos)][d_k]`` float32 holding values of the workload's dtype."""
    return global_rows(case.seed, TENSOR_DOUT, case.h_q, case.d_k, q_pos, 1.0,
                       case.dtype == "bf16")


TENSOR_DOCS = 4


def document_starts(T, seed, min_len=512, max_len=32768):
    """First global positions of the documents packed into a T-token sequence.

    Packed-sequence recipe: document lengths are drawn log-uniformly between
    ``min_len`` and ``max_len`` tokens from
    ``numpy.random.Generator(PCG64(SeedSequence([seed, 4])))`` and laid end to
    end from position 0; the last document is cut at T.  Returns an
    increasing int64 array whose first entry is 0.
    """
    if T <= 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TENSOR_DOCS])))
    starts = [0]
    lo, hi = np.log(min_len), np.log(max_len)
    while True:
        n = int(round(float(np.exp(rng.uniform(lo, hi)))))
        nxt = starts[-1] + max(1, n)
        if nxt >= T:
            break
        starts.append(nxt)
    return np.asarray(starts, dtype=np.int64)

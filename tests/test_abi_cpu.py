"""The C-ABI library without a GPU: it loads, exports every symbol that
include/ra.h declares, and rejects bad arguments on the host before any
device work (these calls never reach the HIP runtime)."""

import ctypes
import os
import re

import pytest

import torch

import ring_attention_rank_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ra.LIB_PATH), reason="libra.so not built")

OK, NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, HIP, ARG = 0, -1, -2, -3, -4, -5, -6, -7
FAKE = 1 << 40  # an aligned address that is never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(ra_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(ra.SYMBOLS)
    L = ra.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.ra_abi_version() == 1


def test_status_strings():
    for s in (OK, NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, HIP, ARG):
        assert ra.status_string(s)
    assert ra.status_string(12345) == "unknown status"


def good(**kw):
    d = dict(n_q=256, n_k=256, h_q=4, h_kv=2, d_k=128, dtype=ra.RA_BF16, causal=True, scale=None)
    d.update(kw)
    return ra.problem(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(h_q=3, h_kv=2), SHAPE),
    (dict(d_k=96), SHAPE),
    (dict(n_q=-1), SHAPE),
    (dict(h_q=0), SHAPE),
    (dict(h_q=512, h_kv=1), SHAPE),
    (dict(n_k=(1 << 23)), SHAPE),                     # one head's block at 2 GiB (bf16, d 128)
    (dict(n_q=(1 << 22), dtype=torch.float32), SHAPE),  # one head's queries at 2 GiB (fp32)
    (dict(dtype=7), DTYPE),
    (dict(scale=-1.0), ARG),
    (dict(scale=float("inf")), ARG),
])
def test_bad_problem(kw, status):
    p = good(**kw)
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    assert ra.lib().ra_tile_shape(ctypes.byref(p), ctypes.byref(bm), ctypes.byref(bn)) == status
    assert ra.lib().ra_forward_workspace_bytes(ctypes.byref(p)) == 0
    v = ctypes.c_void_p(FAKE)
    assert ra.lib().ra_step(ctypes.byref(p), v, v, v, v, v, v, v, v, None, None) == status


def test_null_problem():
    v = ctypes.c_void_p(FAKE)
    assert ra.lib().ra_step(None, v, v, v, v, v, v, v, v, None, None) == NULL
    assert ra.lib().ra_state_init(None, v, v, v, None) == NULL


def test_tile_shape_and_workspace():
    p = good()
    assert ra.tile_shape(p) == (32, 64)
    n = ra.workspace_bytes(p)
    # 2 states (m, l, o in fp32: the two chains') + 4 slots of K, V (bf16)
    # and positions (two blocks read, the next two arriving)
    state = 4 * 256 * 4 * 2 + 4 * 256 * 128 * 4
    slots = 4 * (2 * 2 * 256 * 128 * 2 + 256 * 4)
    assert 2 * state + slots <= n <= 2 * state + slots + 16 * 256
    # other shapes: 2 slots (fp32 K, V)
    nf = ra.workspace_bytes(good(dtype=ra.RA_F32))
    fslots = 2 * (2 * 2 * 256 * 128 * 4 + 256 * 4)
    assert state + fslots <= nf <= state + fslots + 16 * 256


def test_step_pointer_checks():
    p = good()
    v = ctypes.c_void_p(FAKE)
    z = ctypes.c_void_p(0)
    L = ra.lib()
    assert L.ra_step(ctypes.byref(p), z, v, v, v, v, v, v, v, None, None) == NULL
    assert L.ra_step(ctypes.byref(p), v, v, v, z, v, v, v, v, None, None) == NULL
    odd = ctypes.c_void_p(FAKE + 8)
    assert L.ra_step(ctypes.byref(p), odd, v, v, v, v, v, v, v, None, None) == ALIGN
    assert L.ra_step(ctypes.byref(p), v, v, odd, v, v, v, v, v, None, None) == ALIGN
    assert L.ra_step(ctypes.byref(p), v, v, v, v, v, v, v, odd, None, None) == ALIGN
    assert L.ra_step(ctypes.byref(p), v, ctypes.c_void_p(FAKE + 2), v, v, v, v, v, v, None, None) == ALIGN


def test_forward_checks():
    p = good()
    L = ra.lib()
    v = ctypes.c_void_p(FAKE)
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    staged = ctypes.c_int64(0)
    need = ra.workspace_bytes(p)
    args = lambda ncp, ws, wsb: (ctypes.byref(p), ncp, v, v, arr, arr, arr, ws, wsb, v, v,
                                 None, ctypes.byref(staged), None, None)
    assert L.ra_forward(*args(0, v, need)) == SHAPE
    assert L.ra_forward(*args(2, v, need - 1)) == WORKSPACE
    assert L.ra_forward(*args(2, ctypes.c_void_p(0), need)) == NULL
    assert L.ra_forward(*args(2, ctypes.c_void_p(FAKE + 4), need)) == ALIGN
    bad = (ctypes.c_void_p * 2)(FAKE, 0)
    assert L.ra_forward(ctypes.byref(p), 2, v, v, bad, arr, arr, v, need, v, v, None,
                        ctypes.byref(staged), None, None) == NULL


def test_forward_timed_checks():
    """ra_forward_timed checks what ra_forward checks, and every event handle
    it is given, before enqueuing anything."""
    p = good()
    L = ra.lib()
    v = ctypes.c_void_p(FAKE)
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    staged = ctypes.c_int64(0)
    need = ra.workspace_bytes(p)
    launch = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, 0)
    cps = (ctypes.c_void_p * 2)(0, FAKE)
    args = lambda ncp, ws, wsb: (ctypes.byref(p), ncp, v, v, arr, arr, arr, ws, wsb, v, v,
                                 None, ctypes.byref(staged), None, None)
    assert L.ra_forward_timed(*args(0, v, need), None, None) == SHAPE
    assert L.ra_forward_timed(*args(2, v, need - 1), None, None) == WORKSPACE
    assert L.ra_forward_timed(*args(2, v, need), launch, None) == NULL
    assert L.ra_forward_timed(*args(2, v, need), None, cps) == NULL


def test_forward_noalloc_refuses_oversize():
    """A share whose workspace exceeds RA_NOALLOC_MAX_BYTES is refused before
    any device call; a bad problem reports its own error."""
    L = ra.lib()
    v = ctypes.c_void_p(FAKE)
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    big = good(n_q=8192, h_q=64, h_kv=1)
    assert ra.workspace_bytes(big) > ra.NOALLOC_MAX_BYTES
    args = lambda p: (ctypes.byref(p), 2, v, v, arr, arr, arr, v, v, None, None, None, None)
    assert L.ra_forward_noalloc(*args(big)) == WORKSPACE
    assert L.ra_forward_noalloc(*args(good(d_k=96))) == SHAPE
    # the full 8B share: ra_forward's workspace (two states, four slots)
    # exceeds the array, but the no-alloc form's own (one state, two slots:
    # about 200 MB) fits, so the size check passes (without a device the
    # call then fails on the device query, never on the size)
    p8 = good(n_q=8192, n_k=8192, h_q=32, h_kv=8)
    assert ra.workspace_bytes(p8) > ra.NOALLOC_MAX_BYTES
    if not torch.cuda.is_available():
        assert L.ra_forward_noalloc(*args(p8)) not in (WORKSPACE, SHAPE, NULL, ALIGN)


def test_mfma_ceiling_checks():
    L = ra.lib()
    v = ctypes.c_void_p(FAKE)
    assert L.ra_mfma_ceiling(0, 10, v, None) == SHAPE
    assert L.ra_mfma_ceiling(4, 0, v, None) == SHAPE
    assert L.ra_mfma_ceiling(4, 10, None, None) == NULL
    assert L.ra_mfma_ceiling(4, 10, ctypes.c_void_p(FAKE + 2), None) == ALIGN


def test_debug_position_check(monkeypatch):
    """RA_DEBUG=1 makes the binding refuse positions that do not increase and
    document starts that decrease; without it nothing is checked."""
    up = torch.tensor([0, 3, 7], dtype=torch.int32)
    flat = torch.tensor([0, 3, 3], dtype=torch.int32)
    down = torch.tensor([5, 2, 2], dtype=torch.int32)
    ra._check_increasing(flat, [flat], down)
    monkeypatch.setenv("RA_DEBUG", "1")
    ra._check_increasing(up, [up], torch.tensor([0, 0, 4], dtype=torch.int32))
    with pytest.raises(ValueError):
        ra._check_increasing(flat, [up])
    with pytest.raises(ValueError):
        ra._check_increasing(up, [up, flat])
    with pytest.raises(ValueError):
        ra._check_increasing(up, [up], down)


def test_allgather_checks():
    L = ra.lib()
    v = ctypes.c_void_p(FAKE)
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    p = good()  # bf16, d_k 128: the register-resident path needs no workspace
    assert ra.allgather_workspace_bytes(p) == 0
    args = lambda p, ncp, ws, wsb: (ctypes.byref(p), ncp, v, v, arr, arr, arr, ws, wsb, v, v,
                                    None, None)
    assert L.ra_forward_allgather(*args(p, 0, None, 0)) == SHAPE
    assert L.ra_forward_allgather(*args(p, 65, None, 0)) == SHAPE
    bad = (ctypes.c_void_p * 2)(FAKE, 0)
    assert L.ra_forward_allgather(ctypes.byref(p), 2, v, v, arr, bad, arr, None, 0, v, v,
                                  None, None) == NULL
    odd = (ctypes.c_void_p * 2)(FAKE, FAKE + 8)
    assert L.ra_forward_allgather(ctypes.byref(p), 2, v, v, odd, arr, arr, None, 0, v, v,
                                  None, None) == ALIGN
    # one to two work units per compute unit (256 on a device with 256
    # compute units, the count assumed without a device): two partial states
    # for the two chains
    pc = good(n_q=2048, h_q=32, h_kv=8)
    assert ra.allgather_workspace_bytes(pc) >= 2 * (32 * 2048 * 4 * 2 + 32 * 2048 * 128 * 4)
    # other shapes keep the running state in the workspace
    pf = ra.problem(256, 256, 4, 2, 64, torch.float32)
    need = ra.allgather_workspace_bytes(pf)
    assert need >= 4 * 256 * 4 * 2 + 4 * 256 * 64 * 4
    assert L.ra_forward_allgather(*args(pf, 2, None, need)) == NULL
    assert L.ra_forward_allgather(*args(pf, 2, v, need - 1)) == WORKSPACE
    assert L.ra_forward_allgather(*args(pf, 2, ctypes.c_void_p(FAKE + 4), need)) == ALIGN


def test_allgather_docs_checks():
    """The document-masked all-gather entry point refuses, before any device
    work, a non-causal problem, a missing or misaligned document-start array,
    and whatever ra_forward_allgather refuses."""
    L = ra.lib()
    v = ctypes.c_void_p(FAKE)
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    p = good()
    call = lambda p, ncp, docs: L.ra_forward_allgather_docs(
        ctypes.byref(p), ncp, v, v, docs, arr, arr, arr, None, 0, v, v, None)
    assert call(good(causal=0), 2, v) == ARG
    assert call(p, 2, None) == NULL
    assert call(p, 2, ctypes.c_void_p(FAKE + 2)) == ALIGN
    assert call(p, 0, v) == SHAPE
    assert call(p, 65, v) == SHAPE
    bad = (ctypes.c_void_p * 2)(FAKE, 0)
    assert L.ra_forward_allgather_docs(ctypes.byref(p), 2, v, v, v, arr, bad, arr, None, 0, v, v,
                                       None) == NULL


def test_allgather_docs_workspace():
    """The document-masked form splits the key blocks of a small launch
    (fewer than 1024 workgroups) over up to one workgroup per block and keeps
    the partial states (m, l, o: 130 floats a row and split) in the workspace;
    a large launch, a single block or the fp32 path does not split."""
    L = ra.lib()
    v = ctypes.c_void_p(FAKE)
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    p = good()  # 2 query tiles x 4 heads: one workgroup pair per head
    rows = 4 * 256
    need2 = ra.allgather_docs_workspace_bytes(p, 2)
    assert need2 >= 2 * rows * 130 * 4
    assert ra.allgather_docs_workspace_bytes(p, 4) >= 4 * rows * 130 * 4 > need2
    assert ra.allgather_docs_workspace_bytes(p, 1) == 0
    assert ra.allgather_docs_workspace_bytes(p, 0) == 0
    assert ra.allgather_docs_workspace_bytes(p, 65) == 0
    assert ra.allgather_docs_workspace_bytes(good(d_k=96), 2) == 0
    # 128 query tiles x 16 heads = 1024 workgroups: no split
    assert ra.allgather_docs_workspace_bytes(good(n_q=16384, h_q=16, h_kv=1), 16) == 0
    pf = good(dtype=ra.RA_F32, d_k=64)
    assert ra.allgather_docs_workspace_bytes(pf, 2) == ra.allgather_workspace_bytes(pf) > 0
    call = lambda ws, wsb: L.ra_forward_allgather_docs(ctypes.byref(p), 2, v, v, v, arr, arr, arr,
                                                       ws, wsb, v, v, None)
    assert call(None, need2) == NULL
    assert call(v, need2 - 1) == WORKSPACE
    assert call(ctypes.c_void_p(FAKE + 4), need2) == ALIGN


@pytest.mark.parametrize("n_q,h_q,h_kv,n_cp,splits", [
    (8192, 8, 1, 16, 8),     # 70B stage share: 256 workgroups -> 8 splits
    (8192, 16, 1, 16, 4),    # 405B stage share: 512 -> 4
    (8192, 8, 8, 64, 8),     # striped share: 256 -> 8 (of 64 blocks)
    (8192, 32, 8, 4, 0),     # 8B share: 1024 workgroups, no split
    (256, 4, 2, 3, 3),       # tiny: at most one split per block
])
def test_docs_split_counts(n_q, h_q, h_kv, n_cp, splits):
    """The split count behind the document-masked workspace: about 2048
    workgroups for launches under 1024, at most one split per block; the
    workspace holds 130 floats per row and split (plus alignment)."""
    p = good(n_q=n_q, n_k=n_q, h_q=h_q, h_kv=h_kv)
    ws = ra.allgather_docs_workspace_bytes(p, n_cp)
    per_split = h_q * n_q * 130 * 4
    assert ws // per_split == splits
    assert ws - splits * per_split < 3 * 256
    # the count the library reports itself (1 = no split)
    assert ra.docs_splits(p, n_cp) == max(splits, 1)


def test_docs_split_span_and_bad_arguments():
    assert ra.docs_split_span() == 8192
    assert ra.docs_splits(good(), 0) == 0 and ra.docs_splits(good(), 65) == 0
    assert ra.docs_splits(good(d_k=96), 2) == 0
    assert ra.docs_splits(good(dtype=ra.RA_F32, d_k=64), 4) == 1


def test_backward_checks():
    L = ra.lib()
    v = ctypes.c_void_p(FAKE)
    odd = ctypes.c_void_p(FAKE + 4)
    step = lambda p, *ptrs: L.ra_backward_step(ctypes.byref(p), *ptrs, v, 1 << 40, None)
    full = [v] * 11
    # every shape the forward takes (fp32 and d_k 64 run the plain kernels):
    # accepted up to the pointer checks; other shapes refused
    assert step(good(dtype=ra.RA_F32), None, *full[1:]) == NULL
    assert step(good(d_k=64), None, *full[1:]) == NULL
    assert step(good(d_k=96), *full) == SHAPE
    assert step(good(h_q=3), *full) == SHAPE
    assert step(good(dtype=7), *full) == DTYPE
    assert L.ra_backward_prep(ctypes.byref(good(dtype=ra.RA_F32)), None, v, v, None) == NULL
    assert L.ra_backward_prep(ctypes.byref(good(d_k=96)), v, v, v, None) == SHAPE
    # every pointer of a non-empty side is required
    for i in range(11):
        ptrs = list(full)
        ptrs[i] = None
        assert step(good(), *ptrs) == NULL, i
    # q, k, v, dout, dq, dk, dv 16-byte aligned; positions, lse, delta 4-byte
    for i in (0, 2, 3, 5, 8, 9, 10):
        ptrs = list(full)
        ptrs[i] = odd
        assert step(good(), *ptrs) == ALIGN, i
    # nothing to do: no pointer is needed (the empty sides run on the GPU tests)
    assert step(good(n_q=0, n_k=0), *([None] * 11)) == OK
    assert L.ra_backward_prep(ctypes.byref(good()), None, v, v, None) == NULL
    assert L.ra_backward_prep(ctypes.byref(good()), v, odd, v, None) == ALIGN
    assert L.ra_backward_prep(ctypes.byref(good(n_q=0)), None, None, None, None) == OK
    # a head group split across workgroups needs the workspace
    p = good(n_k=8192, h_q=16, h_kv=1)
    need = L.ra_backward_workspace_bytes(ctypes.byref(p))
    assert need > 0 and need % (2 * 8192 * 128 * 4) == 0
    assert L.ra_backward_workspace_bytes(ctypes.byref(good(n_k=8192, h_q=8, h_kv=8))) == 0
    assert L.ra_backward_workspace_bytes(ctypes.byref(good(dtype=ra.RA_F32))) == 0
    ws = lambda w, b: L.ra_backward_step(ctypes.byref(p), *full, w, b, None)
    assert ws(None, need) == NULL
    assert ws(v, need - 1) == WORKSPACE
    assert ws(odd, need) == ALIGN


def test_backward_share_checks():
    L = ra.lib()
    v = ctypes.c_void_p(FAKE)
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    p = good(n_k=8192, h_q=16, h_kv=1)
    need = L.ra_backward_share_workspace_bytes(ctypes.byref(p))
    # delta (h_q x n_q floats) plus the head-group partials of one block
    assert need >= 16 * 256 * 4 + L.ra_backward_workspace_bytes(ctypes.byref(p))
    call = lambda p, ncp, ka, dka, ws, wsb: L.ra_backward_share(
        ctypes.byref(p), ncp, v, v, ka, arr, arr, v, v, v, v, dka, arr, ws, wsb, None, None)
    assert call(p, 0, arr, arr, v, need) == SHAPE
    assert call(p, 2, None, arr, v, need) == NULL
    assert call(p, 2, arr, None, v, need) == NULL
    bad = (ctypes.c_void_p * 2)(FAKE, 0)
    assert call(p, 2, arr, bad, v, need) == NULL
    odd = (ctypes.c_void_p * 2)(FAKE, FAKE + 4)
    assert call(p, 2, arr, odd, v, need) == ALIGN
    assert call(p, 2, arr, arr, None, need) == NULL
    assert call(p, 2, arr, arr, v, need - 1) == WORKSPACE
    assert call(p, 2, arr, arr, ctypes.c_void_p(FAKE + 4), need) == ALIGN
    assert call(good(d_k=96), 2, arr, arr, v, need) == SHAPE


def test_binding_checks_row_arrays():
    """The binding refuses what the C ABI cannot see (before it touches a
    GPU): short or mistyped position arrays and mismatched key/value blocks."""
    q = torch.zeros(2, 8, 64)
    k = torch.zeros(1, 5, 64)
    ok = dict(q=q, q_pos=torch.zeros(8, dtype=torch.int32), k_blocks=[k], v_blocks=[k],
              k_pos_blocks=[torch.zeros(5, dtype=torch.int32)])
    ra._check_rows(**ok)
    bad = [dict(q_pos=torch.zeros(7, dtype=torch.int32)),
           dict(q_pos=torch.zeros(8, dtype=torch.int64)),
           dict(k_pos_blocks=[torch.zeros(4, dtype=torch.int32)]),
           dict(v_blocks=[torch.zeros(1, 6, 64)]),
           dict(k_blocks=[torch.zeros(1, 5, 64, dtype=torch.bfloat16)],
                v_blocks=[torch.zeros(1, 5, 64, dtype=torch.bfloat16)]),
           dict(q_doc_start=torch.zeros(3, dtype=torch.int32))]
    for b in bad:
        with pytest.raises(ValueError):
            ra._check_rows(**{**ok, **b})

"""Python binding of the ring-attention rank-share library (libra.so).

This layer only marshals arguments: torch tensors become device pointers and
torch streams become hipStream_t handles; every step of the computation runs
in the library's HIP kernels.  There is no CPU fallback: when libra.so is
missing or the device is not a GPU, calls raise.

Entry points mirror include/ra.h: ``state_init``, ``step``, ``finalize``,
``forward``, ``forward_allgather``, ``backward_prep``, ``backward_step``,
``backward``, ``tile_shape``, ``workspace_bytes``.
"""

import ctypes
import math
import os

import torch

from . import layouts  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libra.so")

RA_BF16, RA_F32 = 0, 1

SYMBOLS = (
    "ra_state_init", "ra_step", "ra_finalize", "ra_forward_workspace_bytes", "ra_forward",
    "ra_forward_timed", "ra_forward_noalloc",
    "ra_forward_allgather_workspace_bytes", "ra_forward_allgather",
    "ra_forward_allgather_docs_workspace_bytes", "ra_forward_allgather_docs",
    "ra_backward_prep", "ra_backward_workspace_bytes", "ra_backward_step",
    "ra_backward_share_workspace_bytes", "ra_backward_share", "ra_tile_shape", "ra_status_string", "ra_abi_version",
    "ra_docs_split_span", "ra_docs_splits", "ra_mfma_ceiling",
)


class Problem(ctypes.Structure):
    _fields_ = [
        ("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32), ("h_q", ctypes.c_int32),
        ("h_kv", ctypes.c_int32), ("d_k", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
    ]


class RAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib():
    """Load libra.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m ring_attention_rank_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
    P = ctypes.POINTER(Problem)
    L.ra_state_init.argtypes = [P, vp, vp, vp, vp]
    L.ra_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, i64p, vp]
    L.ra_finalize.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.ra_forward_workspace_bytes.argtypes = [P]
    L.ra_forward_workspace_bytes.restype = ctypes.c_size_t
    L.ra_forward.argtypes = [P, i32, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                             ctypes.POINTER(vp), vp, ctypes.c_size_t, vp, vp, vp,
                             ctypes.POINTER(ctypes.c_int64), vp, vp]
    L.ra_forward_timed.argtypes = L.ra_forward.argtypes + [ctypes.POINTER(vp), ctypes.POINTER(vp)]
    L.ra_forward_noalloc.argtypes = [P, i32, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                     ctypes.POINTER(vp), vp, vp, vp,
                                     ctypes.POINTER(ctypes.c_int64), vp, vp]
    L.ra_forward_allgather_workspace_bytes.argtypes = [P]
    L.ra_forward_allgather_workspace_bytes.restype = ctypes.c_size_t
    L.ra_forward_allgather_docs_workspace_bytes.argtypes = [P, i32]
    L.ra_forward_allgather_docs_workspace_bytes.restype = ctypes.c_size_t
    L.ra_forward_allgather.argtypes = [P, i32, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                       ctypes.POINTER(vp), vp, ctypes.c_size_t, vp, vp, vp, vp]
    L.ra_forward_allgather_docs.argtypes = [P, i32, vp, vp, vp, ctypes.POINTER(vp),
                                            ctypes.POINTER(vp), ctypes.POINTER(vp), vp,
                                            ctypes.c_size_t, vp, vp, vp]
    L.ra_backward_prep.argtypes = [P, vp, vp, vp, vp]
    L.ra_backward_workspace_bytes.argtypes = [P]
    L.ra_backward_workspace_bytes.restype = ctypes.c_size_t
    L.ra_backward_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   ctypes.c_size_t, vp]
    L.ra_backward_share_workspace_bytes.argtypes = [P]
    L.ra_backward_share_workspace_bytes.restype = ctypes.c_size_t
    L.ra_backward_share.argtypes = [P, i32, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                    ctypes.POINTER(vp), vp, vp, vp, vp, ctypes.POINTER(vp),
                                    ctypes.POINTER(vp), vp, ctypes.c_size_t, vp, vp]
    L.ra_tile_shape.argtypes = [P, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.ra_status_string.argtypes = [i32]
    L.ra_status_string.restype = ctypes.c_char_p
    L.ra_abi_version.argtypes = []
    L.ra_mfma_ceiling.argtypes = [i32, i32, vp, vp]
    L.ra_mfma_ceiling.restype = i32
    L.ra_docs_split_span.argtypes = []
    L.ra_docs_split_span.restype = i32
    L.ra_docs_splits.argtypes = [P, i32]
    L.ra_docs_splits.restype = i32
    for name in ("ra_state_init", "ra_step", "ra_finalize", "ra_forward", "ra_forward_timed",
                 "ra_forward_noalloc",
                 "ra_tile_shape",
                 "ra_forward_allgather", "ra_forward_allgather_docs", "ra_backward_prep",
                 "ra_backward_step",
                 "ra_backward_share",
                 "ra_abi_version"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def status_string(status):
    return lib().ra_status_string(int(status)).decode()


def _check(status, where):
    if status != 0:
        raise RAError(status, where)


def problem(n_q, n_k, h_q, h_kv, d_k, dtype, causal=True, scale=None):
    """Build the ra_problem struct.  ``dtype`` is a torch dtype or RA_* code."""
    if isinstance(dtype, torch.dtype):
        dtype = {torch.bfloat16: RA_BF16, torch.float32: RA_F32}.get(dtype, -1)
    return Problem(int(n_q), int(n_k), int(h_q), int(h_kv), int(d_k), int(dtype),
                   1 if causal else 0, 0.0 if scale is None else float(scale))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _stream(s=None):
    if s is None:
        s = torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need_gpu(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _check_rows(q, q_pos, k_blocks, v_blocks, k_pos_blocks, q_doc_start=None):
    """What the C ABI cannot see: each position array is an int32 vector
    with one entry per row, and every key/value block has the first block's
    shape and q's element type.  Kernels read positions by row index, so a
    short array would be read past its end."""
    if q.dim() != 3:
        raise ValueError("q must be [h_q][n_q][d_k]")
    n_q, d_k = q.shape[1], q.shape[2]

    def vec(t, n, name):
        if t.dtype != torch.int32 or t.dim() != 1 or t.numel() != n:
            raise ValueError(f"{name} must be an int32 vector of {n} positions")

    vec(q_pos, n_q, "q_pos")
    if q_doc_start is not None:
        vec(q_doc_start, n_q, "q_doc_start")
    shape = tuple(k_blocks[0].shape)
    if len(shape) != 3 or shape[2] != d_k:
        raise ValueError("key/value blocks must be [h_kv][n_k][d_k] with q's d_k")
    for k, v, kp in zip(k_blocks, v_blocks, k_pos_blocks):
        if tuple(k.shape) != shape or tuple(v.shape) != shape or k.dtype != q.dtype \
                or v.dtype != q.dtype:
            raise ValueError("every key/value block needs the first block's shape and q's dtype")
        vec(kp, shape[1], "k_pos")
    _check_increasing(q_pos, k_pos_blocks, q_doc_start)


def _check_increasing(q_pos, k_pos_blocks, q_doc_start=None):
    """With RA_DEBUG=1 in the environment: positions must increase strictly
    within each array, and document starts must not decrease (the kernels'
    tile classes rely on both; otherwise the values are unspecified).  The
    check synchronises with the device, so it is off by default."""
    if os.environ.get("RA_DEBUG", "0") in ("", "0"):
        return
    for name, t in [("q_pos", q_pos)] + [(f"k_pos[{b}]", kp) for b, kp in enumerate(k_pos_blocks)]:
        if t.numel() > 1 and not bool((t[1:] > t[:-1]).all()):
            raise ValueError(f"{name}: positions must increase strictly")
    if q_doc_start is not None and q_doc_start.numel() > 1 \
            and not bool((q_doc_start[1:] >= q_doc_start[:-1]).all()):
        raise ValueError("q_doc_start must not decrease")


def _problem_from(q, k, causal, scale):
    h_q, n_q, d_k = q.shape
    h_kv, n_k, _ = k.shape
    return problem(n_q, n_k, h_q, h_kv, d_k, q.dtype, causal, scale)


def tile_shape(p):
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().ra_tile_shape(ctypes.byref(p), ctypes.byref(bm), ctypes.byref(bn)), "ra_tile_shape")
    return bm.value, bn.value


def workspace_bytes(p):
    return int(lib().ra_forward_workspace_bytes(ctypes.byref(p)))


def new_state(h_q, n_q, d_k, device):
    m = torch.empty((h_q, n_q), dtype=torch.float32, device=device)
    l = torch.empty((h_q, n_q), dtype=torch.float32, device=device)
    o = torch.empty((h_q, n_q, d_k), dtype=torch.float32, device=device)
    return m, l, o


def state_init(p, m, l, o, stream=None):
    _need_gpu(m, l, o)
    _check(lib().ra_state_init(ctypes.byref(p), _ptr(m), _ptr(l), _ptr(o), _stream(stream)),
           "ra_state_init")


def step(q, q_pos, k, v, k_pos, m, l, o, work=None, causal=True, scale=None, stream=None):
    """Fold one key/value block into the state (m, l, o) in place."""
    _need_gpu(q, q_pos, k, v, k_pos, m, l, o, work)
    _check_rows(q, q_pos, [k], [v], [k_pos])
    p = _problem_from(q, k, causal, scale)
    _check(lib().ra_step(ctypes.byref(p), _ptr(q), _ptr(q_pos), _ptr(k), _ptr(v), _ptr(k_pos),
                         _ptr(m), _ptr(l), _ptr(o), _ptr(work), _stream(stream)), "ra_step")


def finalize(p, m, l, o, out=None, lse=None, stream=None):
    _need_gpu(m, l, o)
    if out is None:
        out = torch.empty_like(o)
    if lse is None:
        lse = torch.empty_like(m)
    _need_gpu(out, lse)
    _check(lib().ra_finalize(ctypes.byref(p), _ptr(m), _ptr(l), _ptr(o), _ptr(out), _ptr(lse),
                             _stream(stream)), "ra_finalize")
    return out, lse


_side_streams = {}


def side_stream(device=None):
    """A per-device side stream (default priority) for ring staging copies."""
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else device) \
        if not isinstance(device, torch.device) else device
    s = _side_streams.get(dev.index)
    if s is None:
        s = torch.cuda.Stream(device=dev)
        _side_streams[dev.index] = s
    return s


def _record_streams(obj, streams, tensors):
    """The buffers of a prepared call were allocated on the stream current at
    its construction; work enqueued on another stream (the caller's, or the
    side stream that fills staging slots) must keep them alive until it has
    run, so the caching allocator is told of each such stream once."""
    for st in streams:
        if st is None or st.cuda_stream == obj.alloc_stream.cuda_stream \
                or st.cuda_stream in obj.recorded:
            continue
        for t in tensors:
            if t is not None:
                t.record_stream(st)
        obj.recorded.add(st.cuda_stream)


class Forward:
    """A prepared ra_forward call: the pointer arrays, workspace and outputs
    are built once, so repeated calls only cross the C ABI."""

    def __init__(self, q, q_pos, k_blocks, v_blocks, k_pos_blocks, causal=True, scale=None,
                 side=True, count_work=True, workspace=None):
        _need_gpu(q, q_pos, *k_blocks, *v_blocks, *k_pos_blocks)
        n_cp = len(k_blocks)
        if not (n_cp == len(v_blocks) == len(k_pos_blocks)) or n_cp < 1:
            raise ValueError("need n_cp >= 1 blocks of k, v and k_pos")
        _check_rows(q, q_pos, k_blocks, v_blocks, k_pos_blocks)
        self.p = _problem_from(q, k_blocks[0], causal, scale)
        self.n_cp = n_cp
        dev = q.device
        self.keep = (q, q_pos, list(k_blocks), list(v_blocks), list(k_pos_blocks))
        arr = ctypes.c_void_p * n_cp
        self.kp = arr(*[t.data_ptr() for t in k_blocks])
        self.vp = arr(*[t.data_ptr() for t in v_blocks])
        self.pp = arr(*[t.data_ptr() for t in k_pos_blocks])
        nbytes = workspace_bytes(self.p)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        self.ws = workspace
        self.out = torch.empty(q.shape, dtype=torch.float32, device=dev)
        self.lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        self.work = torch.zeros(3, dtype=torch.int64, device=dev) if count_work else None
        self.side = side_stream(dev) if side else None
        self.staged = ctypes.c_int64(0)
        self.alloc_stream = torch.cuda.current_stream(dev)
        self.recorded = set()

    def _mark_streams(self, main):
        _record_streams(self, (main, self.side), (self.ws, self.out, self.lse, self.work))

    def __call__(self, stream=None):
        return self._run(stream, None, None)

    def _run(self, stream, launch_events, staged_events):
        main = torch.cuda.current_stream() if stream is None else stream
        side = self.side if self.side is not None else None
        self._mark_streams(main)
        q, q_pos = self.keep[0], self.keep[1]
        args = (ctypes.byref(self.p), self.n_cp, _ptr(q), _ptr(q_pos), self.kp, self.vp, self.pp,
                _ptr(self.ws), ctypes.c_size_t(self.ws.numel()), _ptr(self.out), _ptr(self.lse),
                _ptr(self.work), ctypes.byref(self.staged), _stream(main),
                ctypes.c_void_p(side.cuda_stream) if side is not None else ctypes.c_void_p(0))
        if launch_events is None and staged_events is None:
            _check(lib().ra_forward(*args), "ra_forward")
        else:
            _check(lib().ra_forward_timed(*args, launch_events, staged_events), "ra_forward_timed")
        return self.out, self.lse

    def timed(self, stream=None):
        """One call of ra_forward_timed, synchronised: per step b the kernel
        time (ms between the marks around its launch), the gap since step
        b-1 ended, and the exposed staging wait, i.e. how long after step b-1
        ended block b's copies finished (0 when the copy was already done)."""
        main = torch.cuda.current_stream() if stream is None else stream
        n = self.n_cp
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(3 * n)]
        for e in evs:  # torch creates the HIP event on its first record
            e.record(main)
        main.synchronize()
        arr = ctypes.c_void_p * n
        launch = (ctypes.c_void_p * (2 * n))(*[e.cuda_event for e in evs[:2 * n]])
        staged = arr(*[e.cuda_event for e in evs[2 * n:]])
        self._run(main, launch, staged)
        main.synchronize()
        if self.side is not None:
            self.side.synchronize()
        st, en, cp = evs[0:2 * n:2], evs[1:2 * n:2], evs[2 * n:]
        kernel_ms = [st[b].elapsed_time(en[b]) for b in range(n)]
        gap_ms = [0.0] + [en[b - 1].elapsed_time(st[b]) for b in range(1, n)]
        wait_ms = [0.0] + [max(0.0, en[b - 1].elapsed_time(cp[b])) for b in range(1, n)]
        total_ms = cp[0].elapsed_time(en[n - 1])
        return {"kernel_ms": kernel_ms, "gap_ms": gap_ms, "staging_wait_ms": wait_ms,
                "total_ms": total_ms}


NOALLOC_MAX_BYTES = 256 << 20  # RA_NOALLOC_MAX_BYTES of include/ra.h


def forward_noalloc(q, q_pos, k_blocks, v_blocks, k_pos_blocks, out, lse, work=None, causal=True,
                    scale=None, side=True, stream=None):
    """ra_forward_noalloc: the ring forward with the library's fixed per-device
    workspace; ``out`` (fp32 like q) and ``lse`` are the caller's.  Returns
    the staged byte count.  Calls that overlap on one device race."""
    _need_gpu(q, q_pos, *k_blocks, *v_blocks, *k_pos_blocks, out, lse, work)
    n_cp = len(k_blocks)
    if not (n_cp == len(v_blocks) == len(k_pos_blocks)) or n_cp < 1:
        raise ValueError("need n_cp >= 1 blocks of k, v and k_pos")
    _check_rows(q, q_pos, k_blocks, v_blocks, k_pos_blocks)
    if tuple(out.shape) != tuple(q.shape) or out.dtype != torch.float32 \
            or tuple(lse.shape) != tuple(q.shape[:2]) or lse.dtype != torch.float32:
        raise ValueError("out must be float32 like q and lse float32 [h_q][n_q]")
    p = _problem_from(q, k_blocks[0], causal, scale)
    arr = ctypes.c_void_p * n_cp
    main = torch.cuda.current_stream() if stream is None else stream
    sd = side_stream(q.device) if side else None
    staged = ctypes.c_int64(0)
    _check(lib().ra_forward_noalloc(
        ctypes.byref(p), n_cp, _ptr(q), _ptr(q_pos), arr(*[t.data_ptr() for t in k_blocks]),
        arr(*[t.data_ptr() for t in v_blocks]), arr(*[t.data_ptr() for t in k_pos_blocks]),
        _ptr(out), _ptr(lse), _ptr(work), ctypes.byref(staged), _stream(main),
        ctypes.c_void_p(sd.cuda_stream) if sd is not None else ctypes.c_void_p(0)),
        "ra_forward_noalloc")
    return staged.value


class ForwardGraph:
    """ra_forward captured once in a HIP graph and replayed.

    The share's staging copies, the events between the launch and side
    streams, and the n_cp step launches go to the GPU as one graph launch.
    The graph reads the same device buffers on every replay: refresh q, k, v
    and the positions in place, and read the results from ``out`` and
    ``lse`` (overwritten by each replay).  A replay runs on the current stream.
    """

    def __init__(self, q, q_pos, k_blocks, v_blocks, k_pos_blocks, causal=True, scale=None):
        self.fwd = Forward(q, q_pos, k_blocks, v_blocks, k_pos_blocks, causal, scale, side=True,
                           count_work=False)
        self.stream = torch.cuda.Stream(device=q.device)
        self.stream.wait_stream(torch.cuda.current_stream(q.device))
        self.fwd(stream=self.stream)  # one eager call first, outside the capture
        self.stream.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=self.stream):
            self.fwd(stream=self.stream)
        self.out, self.lse = self.fwd.out, self.fwd.lse

    def __call__(self):
        self.graph.replay()  # on the current stream, in order with the caller's work
        return self.out, self.lse


def mfma_ceiling(iters=65536, workgroups_per_cu=4, reps=3, stream=None):
    """Sustained bf16 MFMA rate of this device (TFLOP/s, and the ms of the
    timed call) from ra_mfma_ceiling: four 8-wave workgroups per compute
    unit, about 50 ms a call, timed with HIP events on the launch stream.
    The chip lowers its clock over the first milliseconds of such a load, so
    the last of ``reps`` back-to-back calls is the steady-state figure."""
    dev = torch.cuda.current_device()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    n = cus * workgroups_per_cu
    sink = torch.empty(n, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream() if stream is None else stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for rep in range(reps):
        e0.record(s)
        _check(lib().ra_mfma_ceiling(n, int(iters), _ptr(sink), _stream(s)), "ra_mfma_ceiling")
        e1.record(s)
    s.synchronize()
    ms = e0.elapsed_time(e1)
    flops = n * 8 * 4 * iters * 32768
    return flops / (ms * 1e-3) / 1e12, ms


def docs_split_span():
    """Positions a 128-row query tile may span (first row's document start to
    last row's position) before the document-masked launch splits its walk."""
    return int(lib().ra_docs_split_span())


def docs_splits(p, n_cp):
    """Key-block splits of the document-masked launch for this problem (1 = none)."""
    return int(lib().ra_docs_splits(ctypes.byref(p), int(n_cp)))


def allgather_workspace_bytes(p):
    return int(lib().ra_forward_allgather_workspace_bytes(ctypes.byref(p)))


def allgather_docs_workspace_bytes(p, n_cp):
    return int(lib().ra_forward_allgather_docs_workspace_bytes(ctypes.byref(p), n_cp))


class AllGather:
    """A prepared ra_forward_allgather call (every key/value block resident).
    With ``q_doc_start`` (int32 per query: the first global position of its
    document) it is ra_forward_allgather_docs, the document-masked form,
    which reports no tile counters."""

    def __init__(self, q, q_pos, k_blocks, v_blocks, k_pos_blocks, causal=True, scale=None,
                 count_work=True, q_doc_start=None):
        _need_gpu(q, q_pos, *k_blocks, *v_blocks, *k_pos_blocks,
                  *([] if q_doc_start is None else [q_doc_start]))
        self.q_doc_start = q_doc_start
        if q_doc_start is not None:
            count_work = False
        n_cp = len(k_blocks)
        if not (n_cp == len(v_blocks) == len(k_pos_blocks)) or n_cp < 1:
            raise ValueError("need n_cp >= 1 blocks of k, v and k_pos")
        _check_rows(q, q_pos, k_blocks, v_blocks, k_pos_blocks, q_doc_start)
        self.p = _problem_from(q, k_blocks[0], causal, scale)
        self.n_cp = n_cp
        dev = q.device
        self.keep = (q, q_pos, list(k_blocks), list(v_blocks), list(k_pos_blocks))
        arr = ctypes.c_void_p * n_cp
        self.kp = arr(*[t.data_ptr() for t in k_blocks])
        self.vp = arr(*[t.data_ptr() for t in v_blocks])
        self.pp = arr(*[t.data_ptr() for t in k_pos_blocks])
        nbytes = (allgather_workspace_bytes(self.p) if q_doc_start is None
                  else allgather_docs_workspace_bytes(self.p, n_cp))
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
        self.out = torch.empty(q.shape, dtype=torch.float32, device=dev)
        self.lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        self.work = torch.zeros(3, dtype=torch.int64, device=dev) if count_work else None
        self.alloc_stream = torch.cuda.current_stream(dev)
        self.recorded = set()

    def __call__(self, stream=None):
        if stream is not None:
            _record_streams(self, (stream,), (self.ws, self.out, self.lse, self.work))
        q, q_pos = self.keep[0], self.keep[1]
        ws_n = ctypes.c_size_t(self.ws.numel() if self.ws is not None else 0)
        if self.q_doc_start is None:
            _check(lib().ra_forward_allgather(
                ctypes.byref(self.p), self.n_cp, _ptr(q), _ptr(q_pos), self.kp, self.vp, self.pp,
                _ptr(self.ws), ws_n, _ptr(self.out), _ptr(self.lse), _ptr(self.work),
                _stream(stream)), "ra_forward_allgather")
        else:
            _check(lib().ra_forward_allgather_docs(
                ctypes.byref(self.p), self.n_cp, _ptr(q), _ptr(q_pos), _ptr(self.q_doc_start),
                self.kp, self.vp, self.pp, _ptr(self.ws), ws_n, _ptr(self.out), _ptr(self.lse),
                _stream(stream)), "ra_forward_allgather_docs")
        return self.out, self.lse


def forward_allgather(q, q_pos, k_blocks, v_blocks, k_pos_blocks, causal=True, scale=None,
                      q_doc_start=None):
    """The rank share with every block resident: returns (out, lse, work[3] tensor,
    or None under a document mask given by ``q_doc_start``)."""
    f = AllGather(q, q_pos, k_blocks, v_blocks, k_pos_blocks, causal, scale,
                  q_doc_start=q_doc_start)
    out, lse = f()
    return out, lse, f.work


def forward(q, q_pos, k_blocks, v_blocks, k_pos_blocks, causal=True, scale=None, side=True):
    """One rank's share: returns (out, lse, work[3] tensor, staged_bytes)."""
    f = Forward(q, q_pos, k_blocks, v_blocks, k_pos_blocks, causal, scale, side)
    out, lse = f()
    return out, lse, f.work, f.staged.value


def backward_prep(out, dout, delta=None, stream=None):
    """delta[h_q][n_q] = rowsum(dout * out) (fp32) for the backward; ``out`` is
    the forward's fp32 output, ``dout`` its gradient in the queries' dtype."""
    _need_gpu(out, dout, delta)
    h_q, n_q, d_k = out.shape
    p = problem(n_q, 0, h_q, h_q, d_k, dout.dtype)
    if delta is None:
        delta = torch.empty((h_q, n_q), dtype=torch.float32, device=out.device)
    _check(lib().ra_backward_prep(ctypes.byref(p), _ptr(out), _ptr(dout), _ptr(delta),
                                  _stream(stream)), "ra_backward_prep")
    return delta


def backward_workspace_bytes(p):
    return int(lib().ra_backward_workspace_bytes(ctypes.byref(p)))


def backward_step(q, q_pos, k, v, k_pos, dout, lse, delta, dq, dk=None, dv=None, causal=True,
                  scale=None, stream=None, workspace=None):
    """One key/value block of the backward: adds this block's part to ``dq``,
    ``dk`` and ``dv`` (fp32, in place; dk and dv are zero-filled here when
    None) and returns (dk, dv), fp32 ``[h_kv][n_k][d_k]``.  ``workspace`` is a
    uint8 device tensor of at least ``backward_workspace_bytes`` bytes
    (allocated here when None)."""
    if dk is None:
        dk = torch.zeros(k.shape, dtype=torch.float32, device=k.device)
    if dv is None:
        dv = torch.zeros(v.shape, dtype=torch.float32, device=v.device)
    _need_gpu(q, q_pos, k, v, k_pos, dout, lse, delta, dq, dk, dv, workspace)
    _check_rows(q, q_pos, [k], [v], [k_pos])
    p = _problem_from(q, k, causal, scale)
    if workspace is None:
        need = backward_workspace_bytes(p)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    wsb = workspace.numel() if workspace is not None else 0
    _check(lib().ra_backward_step(ctypes.byref(p), _ptr(q), _ptr(q_pos), _ptr(k), _ptr(v),
                                  _ptr(k_pos), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq),
                                  _ptr(dk), _ptr(dv), _ptr(workspace), wsb, _stream(stream)),
           "ra_backward_step")
    return dk, dv


def backward(q, q_pos, k_blocks, v_blocks, k_pos_blocks, out, lse, dout, causal=True,
             scale=None, stream=None):
    """The rank share's backward over every block: returns (dq, dks, dvs), fp32,
    one (dk, dv) per block in the order given."""
    delta = backward_prep(out, dout, stream=stream)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    dks, dvs = [], []
    need = max([backward_workspace_bytes(_problem_from(q, k, causal, scale)) for k in k_blocks],
               default=0)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    for k, v, kp in zip(k_blocks, v_blocks, k_pos_blocks):
        dk, dv = backward_step(q, q_pos, k, v, kp, dout, lse, delta, dq, causal=causal,
                               scale=scale, stream=stream, workspace=ws)
        dks.append(dk)
        dvs.append(dv)
    return dq, dks, dvs


def backward_share_workspace_bytes(p):
    return int(lib().ra_backward_share_workspace_bytes(ctypes.byref(p)))


class BackwardShare:
    """A prepared whole-share backward (ra_backward_share): outputs and
    workspace allocated once; each call overwrites dq and every block's dk,
    dv with this rank's gradients."""

    def __init__(self, q, q_pos, k_blocks, v_blocks, k_pos_blocks, causal=True, scale=None,
                 side=True):
        self.args = (q, q_pos, list(k_blocks), list(v_blocks), list(k_pos_blocks))
        _need_gpu(q, q_pos, *k_blocks, *v_blocks, *k_pos_blocks)
        _check_rows(q, q_pos, k_blocks, v_blocks, k_pos_blocks)
        self.p = _problem_from(q, k_blocks[0], causal, scale)
        dev = q.device
        self.dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
        self.dks = [torch.empty(k.shape, dtype=torch.float32, device=dev) for k in k_blocks]
        self.dvs = [torch.empty(k.shape, dtype=torch.float32, device=dev) for k in k_blocks]
        need = backward_share_workspace_bytes(self.p)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        self.side = side_stream(dev) if side else None
        n = len(k_blocks)
        arr = lambda ts: (ctypes.c_void_p * n)(*[_ptr(t) for t in ts])
        self.kp, self.vp, self.pp = arr(k_blocks), arr(v_blocks), arr(k_pos_blocks)
        self.dkp, self.dvp = arr(self.dks), arr(self.dvs)
        self.alloc_stream = torch.cuda.current_stream(dev)
        self.recorded = set()

    def __call__(self, out, lse, dout, stream=None):
        q, q_pos = self.args[0], self.args[1]
        _need_gpu(out, lse, dout)
        _record_streams(self, (stream, self.side), (self.dq, self.ws, *self.dks, *self.dvs))
        side = _stream(self.side) if self.side is not None else ctypes.c_void_p(0)
        _check(lib().ra_backward_share(ctypes.byref(self.p), len(self.dks), _ptr(q), _ptr(q_pos),
                                       self.kp, self.vp, self.pp, _ptr(out), _ptr(lse),
                                       _ptr(dout), _ptr(self.dq), self.dkp, self.dvp,
                                       _ptr(self.ws), self.ws.numel(), _stream(stream), side),
               "ra_backward_share")
        return self.dq, self.dks, self.dvs


def backward_share(q, q_pos, k_blocks, v_blocks, k_pos_blocks, out, lse, dout, causal=True,
                   scale=None, side=True):
    """Whole-share backward in one call: returns (dq, dks, dvs), fp32."""
    return BackwardShare(q, q_pos, k_blocks, v_blocks, k_pos_blocks, causal, scale, side)(
        out, lse, dout)

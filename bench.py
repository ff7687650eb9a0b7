"""Benchmark one context-parallel rank's share of causal ring attention on one
MI355X and print one JSON line.

A step is one ra_forward call: state set-up, the n_cp ring steps (each block
after the first staged on a side stream while the previous one computes) and
normalisation, over inputs already resident in HBM.  The metric is visible
causal attention TFLOP/s (4 * d_k * h_q FLOPs per visible query/key pair)
and its fraction of the bf16 MFMA peak.

The default workload is the Llama-3-405B long-context stage share: T=131072,
n_cp=16 zigzag, 16 query heads and 1 key/value head of width 128, bf16, rank 0
(8192 queries against 16 blocks of 8192 keys).
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import ring_attention_rank_amd as ra  # noqa: E402
from ring_attention_rank_amd import comm  # noqa: E402
import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_F32_TFLOPS = 157.3
HBM_GBPS = 8000.0
METRIC = "causal attention TFLOP/s per rank-share and % of bf16 MFMA peak (1 GPU)"


KERNEL_SOURCE = os.path.join(ROOT, "ring_attention_rank_amd", "csrc", "ra_fast.hip")
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_SUMMARY = os.path.join(PROFILES, "traffic_step_kernel_fast_llama405b_stage_share.md")
# The dominant kernel of the ring forward: a middle step (reads and writes the
# running state), n_cp - 2 of the n_cp launches.  G is its groups of 4 waves
# per workgroup: 1 when the launch has at least two query-tile pairs x heads
# per compute unit, else 2 (the library's own rule).


def dominant_kernel(case, n_q, cus):
    n_pairs = ((n_q + 127) // 128 + 1) // 2
    g = 1 if n_pairs * case.h_q >= 2 * cus else 2
    return f"step_kernel_fast<{g}, true, false>"
# The other workloads of the size table timed beside the headline (bf16, d_k=128).
SIDE_WORKLOADS = ("llama8b_gqa_zigzag", "llama70b_stage_share", "million_striped_mha")


def kernel_source_sha256():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def summary_fields(path, workload):
    """The ``- key: value`` lines of a committed profile summary, or None when
    it is missing, covers another workload or predates the kernel source."""
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = dict(re.findall(r"^- ([a-z_0-9]+): (\S+)$", text, re.M))
    if fields.get("workload") != workload or fields.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return fields


def summary_float(path, workload, key):
    fields = summary_fields(path, workload)
    try:
        return float(fields[key]) if fields else None
    except (KeyError, ValueError):
        return None


def committed_traffic(workload):
    """HBM bytes per step launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (calibrated on a plain copy), or None when there is no summary for this
    workload or the kernel source changed since it was taken."""
    return summary_float(TRAFFIC_SUMMARY, workload, "hbm_bytes_per_launch")


def committed_trace_us(workload):
    """Average duration (us) of the dominant kernel in the committed
    rocprofv3 --kernel-trace --stats summary of this workload."""
    return summary_float(os.path.join(PROFILES, f"step_kernel_fast_{workload}.md"), workload,
                         "dominant_avg_us")


def committed_sclk_mhz(workload):
    """Shader clock held during the dominant kernel: GRBM_GUI_ACTIVE per XCD
    over the dispatch's duration, from the committed counter pass."""
    return summary_float(os.path.join(PROFILES, f"mfma_utilisation_{workload}.md"), workload,
                         "sclk_mhz")


def copy_calibration(mib, reps):
    """A plain device-to-device copy of known size, to scale the FETCH_SIZE and
    WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "reps": reps}), flush=True)


def visible_pairs(q_pos, k_pos):
    ks = np.sort(np.asarray(k_pos, dtype=np.int64))
    return int(np.searchsorted(ks, np.asarray(q_pos, dtype=np.int64), side="right").sum())


def long_tiles(q_pos, q_lo, span, rows=128):
    """Query tiles whose last row lies more than ``span`` positions past the
    first row's document start (those the document-masked launch splits)."""
    n = len(q_pos)
    return sum(int(q_pos[min(t + rows, n) - 1] - q_lo[t] > span) for t in range(0, n, rows))


def visible_pairs_docs(q_pos, q_lo, k_pos):
    """Pairs with q_lo[i] <= k_pos[j] <= q_pos[i] (the document mask)."""
    ks = np.sort(np.asarray(k_pos, dtype=np.int64))
    hi = np.searchsorted(ks, np.asarray(q_pos, dtype=np.int64), side="right")
    lo = np.searchsorted(ks, np.asarray(q_lo, dtype=np.int64), side="left")
    return int(np.maximum(hi - lo, 0).sum())


def build_share(case, rank, device):
    L = ra.layouts
    q_pos = L.rank_positions(case.T, case.n_cp, rank, case.layout)
    srcs = [L.ring_block_owner(case.n_cp, rank, b) for b in range(case.n_cp)]
    k_pos = [L.rank_positions(case.T, case.n_cp, s, case.layout) for s in srcs]
    q, kb, vb = synth.case_inputs(case, q_pos, k_pos)
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    gq = torch.from_numpy(q).to(dt).to(device)
    n_cp = case.n_cp
    h_kv, n_k, d = kb[0].shape
    kk = torch.empty((n_cp, h_kv, n_k, d), dtype=dt, device=device)
    vv = torch.empty((n_cp, h_kv, n_k, d), dtype=dt, device=device)
    for b in range(n_cp):
        kk[b].copy_(torch.from_numpy(kb[b]).to(dt))
        vv[b].copy_(torch.from_numpy(vb[b]).to(dt))
    share = dict(q=q, k=kb, v=vb, q_pos=q_pos, k_pos=k_pos, gq=gq,
                 gq_pos=torch.from_numpy(q_pos).to(device),
                 gk=[kk[b] for b in range(n_cp)], gv=[vv[b] for b in range(n_cp)],
                 gk_pos=[torch.from_numpy(p).to(device) for p in k_pos])
    share["pairs_per_step"] = [visible_pairs(q_pos, p) for p in k_pos]
    return share


def cpu_baseline(case, share, out, lse, budget_rows):
    """The float64 oracle on a bounded sample of the same share's query rows
    (every block, same ring order), timed on the host's cores."""
    import oracle  # the CPU baseline is the oracle itself, untuned
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity count
        blas = len(os.sched_getaffinity(0))
    n_q = len(share["q_pos"])
    rows = np.unique(np.linspace(0, n_q - 1, budget_rows).astype(np.int64))
    q = share["q"][:, rows]
    qp = share["q_pos"][rows]
    t0 = time.perf_counter()
    ro, rl = oracle.ring_forward_ref(q, qp, share["k"], share["v"], share["k_pos"])
    dt = time.perf_counter() - t0
    pairs = sum(visible_pairs(qp, p) for p in share["k_pos"])
    flops = 4 * case.d_k * case.h_q * pairs
    idx = torch.from_numpy(rows).to(out.device)
    go = out[:, idx].cpu().numpy().astype(np.float64)
    gl = lse[:, idx].cpu().numpy().astype(np.float64)
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas), "kind": "oracle",
        "sample": f"{len(rows)} of {n_q} query rows (evenly spaced) x {case.h_q} heads against "
                  f"all {case.n_cp} blocks, float64 numpy; {pairs} visible pairs in {dt:.2f} s",
        "seconds": dt,
        "host_cpus": len(os.sched_getaffinity(0)),
        "sample_max_abs_err_out": float(np.abs(go - ro).max()),
        "sample_max_abs_err_lse": float(np.abs(gl - rl).max()),
    }


def time_backward(share, fwd, fwd_flops, steps, warmup, rank):
    """The share's backward in one call (ra_backward_share): delta =
    rowsum(dout * out), then every block's dq kernel on the launch stream and
    its dk/dv kernel on a side stream (the first dq kernel writes dq, dk and
    dv are written: nothing is zeroed).  Its algorithmic flops are five GEMMs
    over the visible pairs (S, dP, dQ, dK, dV), 2.5 times the forward's; the
    dq kernel recomputes S and dP, which is not counted."""
    g = torch.Generator(device="cuda").manual_seed(2024)
    q = share["gq"]
    dout = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    out, lse = fwd.out, fwd.lse
    f = ra.BackwardShare(q, share["gq_pos"], share["gk"], share["gv"], share["gk_pos"], side=True)
    for _ in range(warmup):
        f(out, lse, dout)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        f(out, lse, dout)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    flops = 2.5 * fwd_flops
    n = len(share["gk"])
    split = ra.backward_workspace_bytes(ra._problem_from(q, share["gk"][0], True, None)) > 0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "ms_per_step": dt * 1e3,
            "pct_of_bf16_peak": 100.0 * flops / dt / 1e12 / PEAK_BF16_TFLOPS,
            "flops_per_step": flops, "flops_counted": "S, dP, dQ, dK, dV over visible pairs",
            "entry_point": "ra_backward_share (dk/dv on a side stream)",
            "launches_per_step": 1 + n * (3 if split else 2), "rank": rank}


def launch_timing(fwd, pairs_per_step, case, reps):
    """Per-launch kernel times of the ring forward, measured live: ``reps``
    calls of ra_forward_timed, HIP events recorded on the launch stream right
    before and after every step launch.  Returns the mean time of each step
    launch, the mean gap before it, the exposed staging wait before it and the
    achieved rate of the middle launches (the dominant kernel)."""
    runs = [fwd.timed() for _ in range(reps)]
    n = len(pairs_per_step)
    mean = lambda key: [float(np.mean([r[key][b] for r in runs])) for b in range(n)]
    kern, gap, wait = mean("kernel_ms"), mean("gap_ms"), mean("staging_wait_ms")
    flops = [4 * case.d_k * case.h_q * p for p in pairs_per_step]
    mid = list(range(1, n - 1)) if n > 2 else list(range(n))
    mid_ms = float(np.sum([kern[b] for b in mid]))
    mid_flops = float(np.sum([flops[b] for b in mid]))
    return {
        "reps": reps, "kernel_ms": kern, "gap_ms": gap, "staging_wait_ms": wait,
        "staging_wait_ms_total": float(np.sum(wait)), "gap_ms_total": float(np.sum(gap)),
        "kernel_ms_total": float(np.sum(kern)),
        "forward_ms": float(np.mean([r["total_ms"] for r in runs])),
        "middle_launches": len(mid), "middle_mean_ms": mid_ms / len(mid),
        "middle_flops_per_launch": mid_flops / len(mid),
        "middle_tflops": mid_flops / (mid_ms * 1e-3) / 1e12,
    }


def comm_model(case, staged_bytes, step_ms):
    """The pages' exchange model for this share (Zero to Frontier, "What
    context parallelism communicates" and "When the ring hides its
    communication"): bytes a GPU receives per layer by ring and by Ulysses,
    the group size above which Ulysses moves less, and the link bandwidth a
    real ring would need for one key/value block to arrive within one
    measured step."""
    d, d_kv = case.h_q * case.d_k, case.h_kv * case.d_k
    eb = 2 if case.dtype == "bf16" else 4
    block = comm.kv_block_bytes(case.T // case.n_cp, d_kv, eb)
    ring = comm.cp_comm_bytes(case.T, d, d_kv, case.n_cp, "ring", eb)
    return {
        "ring_bytes_per_layer": ring, "staged_bytes_measured": staged_bytes,
        "ulysses_bytes_per_layer": comm.cp_comm_bytes(case.T, d, d_kv, case.n_cp, "ulysses", eb),
        "ulysses_breakeven_group": comm.ulysses_breakeven(case.h_q, case.h_kv),
        "kv_block_bytes": block, "middle_step_ms": step_ms,
        "link_GBps_to_hide_each_step": block / (step_ms * 1e-3) / 1e9,
    }


def time_ring(case, ranks, dev, steps, warmup, side=True):
    """The headline measure: ``steps`` ra_forward calls per rank share after
    ``warmup`` untimed ones, wall clock with the device synchronised on both
    sides; per-step HIP events on the launch stream alongside."""
    total_flops, total_time, step_ms, per_rank, last = 0, 0.0, [], [], None
    for r in ranks:
        share = build_share(case, r, dev)
        fwd = ra.Forward(share["gq"], share["gq_pos"], share["gk"], share["gv"], share["gk_pos"],
                         side=side)
        flops = 4 * case.d_k * case.h_q * sum(share["pairs_per_step"])
        for _ in range(warmup):
            fwd()
        torch.cuda.synchronize()
        main_stream = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1 in evs:
            e0.record(main_stream)
            fwd()
            e1.record(main_stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [e0.elapsed_time(e1) for e0, e1 in evs]
        step_ms += ms
        total_flops += flops * steps
        total_time += wall
        per_rank.append({"rank": r, "median_ms": float(np.median(ms)),
                         "tflops_median": flops / (np.median(ms) * 1e-3) / 1e12,
                         "visible_flops": flops, "staged_bytes": fwd.staged.value,
                         "work": fwd.work.tolist()})
        last = (share, fwd, flops)
    return {"value": total_flops / total_time / 1e12, "ms_per_step": total_time / (steps * len(ranks)) * 1e3,
            "step_ms": step_ms, "per_rank": per_rank, "last": last}


def time_call(f, steps, warmup):
    """Seconds per call of f (wall clock, device synchronised on both sides)."""
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        f()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def side_workload(name, dev, steps, warmup, timing_reps, cus):
    """One more workload of the size table, timed like the headline: the ring
    forward (every rank share the case lists), its per-launch kernel times
    and staging waits (last rank), and the all-gather form of the last share."""
    case = synth.case_by_name(name)
    ring = time_ring(case, case.ranks, dev, steps, warmup)
    share, fwd, flops = ring.pop("last")
    t = launch_timing(fwd, share["pairs_per_step"], case, timing_reps)
    ag = ra.AllGather(share["gq"], share["gq_pos"], share["gk"], share["gv"], share["gk_pos"])
    ag_s = time_call(ag, steps, warmup)
    out = {
        "value": ring["value"], "unit": "TFLOP/s", "ms_per_step": ring["ms_per_step"],
        "pct_of_bf16_peak": 100.0 * ring["value"] / PEAK_BF16_TFLOPS,
        "config": {"workload": name, "T": case.T, "n_cp": case.n_cp, "layout": case.layout,
                   "ranks": list(case.ranks), "h_q": case.h_q, "h_kv": case.h_kv,
                   "d_k": case.d_k, "n_q": len(share["q_pos"]),
                   "n_k_per_block": len(share["k_pos"][0])},
        "per_rank": ring["per_rank"],
        "dominant_kernel": {
            "kernel": dominant_kernel(case, len(share["q_pos"]), cus),
            "event_mean_ms": t["middle_mean_ms"],
            "achieved": t["middle_tflops"], "frac": t["middle_tflops"] / PEAK_BF16_TFLOPS,
            "traced_avg_us": committed_trace_us(name)},
        "staging_wait_ms_total": t["staging_wait_ms_total"], "gap_ms_total": t["gap_ms_total"],
        "allgather": {"value": flops / ag_s / 1e12, "ms_per_step": ag_s * 1e3,
                      "pct_of_bf16_peak": 100.0 * flops / ag_s / 1e12 / PEAK_BF16_TFLOPS,
                      "rank": case.ranks[-1]},
    }
    tr = out["dominant_kernel"]["traced_avg_us"]
    if tr:
        out["dominant_kernel"]["traced_frac"] = \
            t["middle_flops_per_launch"] / (tr * 1e-6) / 1e12 / PEAK_BF16_TFLOPS
    del fwd, ag, share
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama405b_stage_share",
                    choices=[c.name for c in synth.CASES + synth.ULYSSES_CASES])
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--no-side-stream", action="store_true")
    ap.add_argument("--timing-reps", type=int, default=5,
                    help="ra_forward_timed calls for the per-launch kernel times")
    ap.add_argument("--no-allgather", action="store_true",
                    help="skip timing the all-gather form (every block resident, one launch)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay side line")
    ap.add_argument("--no-docs", action="store_true",
                    help="skip the document-masked all-gather side line")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward of the share (bf16, d_k = 128)")
    ap.add_argument("--no-side-workloads", action="store_true",
                    help="skip timing the other bf16 workloads of the size table")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only run the matrix-pipe calibration (ra_mfma_ceiling) and print it")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's rank share only: the library runs the ring on one "
              "GPU (the exchange between ranks is a copy on that GPU); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return
    if args.mfma_ceiling:
        tf, ms = ra.mfma_ceiling()
        print(json.dumps({"mfma_ceiling_tflops": tf, "ms": ms,
                          "pct_of_bf16_peak": 100.0 * tf / PEAK_BF16_TFLOPS}), flush=True)
        return

    case = synth.case_by_name(args.config)
    ranks = case.ranks if args.rank is None else (args.rank,)
    dev = torch.device("cuda", 0)
    props = torch.cuda.get_device_properties(dev)

    print(f"[bench] ring forward {case.name} ranks {list(ranks)}", file=sys.stderr, flush=True)
    ring = time_ring(case, ranks, dev, args.steps, args.warmup, side=not args.no_side_stream)
    share, fwd, flops = ring["last"]
    value, ms_per_step = ring["value"], ring["ms_per_step"]
    peak = PEAK_BF16_TFLOPS if case.dtype == "bf16" else PEAK_F32_TFLOPS
    n_launch = case.n_cp
    t = launch_timing(fwd, share["pairs_per_step"], case, args.timing_reps)
    fast = case.dtype == "bf16" and case.d_k == 128
    traced_us = committed_trace_us(case.name) if fast else None
    roofline = {
        # achieved: visible FLOPs of a middle ring step over that launch's
        # kernel time, HIP events around each launch on its stream
        "bound": "mfma", "achieved": t["middle_tflops"], "peak": peak, "unit": "TFLOP/s",
        "frac": t["middle_tflops"] / peak, "traffic": committed_traffic(case.name),
        "kernel": (dominant_kernel(case, len(share["q_pos"]), props.multi_processor_count) +
                   " (bf16 MFMA 32x32x16)") if fast else "step_kernel<true, false> (generic)",
        "flops_per_launch": t["middle_flops_per_launch"], "avg_launch_ms": t["middle_mean_ms"],
        "launches_per_step": n_launch, "middle_launches_per_step": t["middle_launches"],
        # the committed kernel trace of the same command (rocprofv3 --stats)
        "traced_avg_us": traced_us,
        "traced_frac": (t["middle_flops_per_launch"] / (traced_us * 1e-6) / 1e12 / peak
                        if traced_us else None),
        # the whole forward per block, gaps between launches included
        "event_forward_per_block_ms": float(np.mean(ring["step_ms"])) / n_launch,
        "event_median_ms_per_step": float(np.median(ring["step_ms"])),
    }
    if fast and not args.no_side_stream:
        n_q = len(share["q_pos"])
        units = ((n_q + 127) // 128 + 1) // 2 * case.h_q
        cus = props.multi_processor_count
        if units >= 2 * cus:
            sched = ("chunk_kernel_fast: launches of two blocks after the first, " if case.n_cp >= 3
                     else "step_kernel_fast: one launch per block, ") + \
                "each as two concurrent half grids (main and side stream)"
        elif units >= cus:
            sched = ("step_kernel_fast<1, ...>: two chains of full-grid launches, even blocks into "
                     "one state on the main stream and odd blocks into another on the side stream, "
                     "merged at the end")
        else:
            sched = ("step_kernel_fast: one launch per block, each as two concurrent half grids "
                     "(main and side stream)")
        roofline["headline_schedule"] = (
            sched + "; the next block(s) staged on the copy stream; the kernel above runs the "
            "same per-tile code, timed alone one launch per block by ra_forward_timed")
    # The bf16 MFMA rate the device sustains with the matrix pipe kept busy and
    # nothing else running: the clock it holds under that load sets it.
    ceil_tf, ceil_ms = ra.mfma_ceiling() if fast else (None, None)
    if ceil_tf:
        roofline["sustained_mfma_tflops"] = ceil_tf
        roofline["frac_of_sustained"] = t["middle_tflops"] / ceil_tf
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {
            "workload": case.name, "T": case.T, "n_cp": case.n_cp, "layout": case.layout,
            "ranks": list(ranks), "h_q": case.h_q, "h_kv": case.h_kv, "d_k": case.d_k,
            "n_q": len(share["q_pos"]), "n_k_per_block": len(share["k_pos"][0]),
            "visible_flops_per_step": flops, "side_stream_staging": not args.no_side_stream,
        },
        "per_rank": ring["per_rank"],
        "roofline": roofline,
        # Zero to Frontier, "When the ring hides its communication": each
        # step's exchange should finish under the previous step's compute.
        "ring_steps": {
            "kernel_ms": t["kernel_ms"], "gap_ms": t["gap_ms"],
            "staging_wait_ms": t["staging_wait_ms"],
            "staging_wait_ms_total": t["staging_wait_ms_total"],
            "gap_ms_total": t["gap_ms_total"], "kernel_ms_total": t["kernel_ms_total"],
            "forward_ms": t["forward_ms"], "reps": t["reps"],
        },
        "comm_model": comm_model(case, fwd.staged.value, t["middle_mean_ms"]),
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "sclk_mhz": committed_sclk_mhz(case.name) if fast else None},
    }
    if not args.no_graph:
        # The same ring forward captured once in a HIP graph and replayed
        # (ra.ForwardGraph): the same copies, events and launches, submitted
        # as one graph launch.  Context only; the headline is the eager call.
        fg = ra.ForwardGraph(share["gq"], share["gq_pos"], share["gk"], share["gv"],
                             share["gk_pos"])
        fg_s = time_call(fg, args.steps, args.warmup)
        result["ring_graph"] = {
            "value": flops / fg_s / 1e12, "unit": "TFLOP/s", "ms_per_step": fg_s * 1e3,
            "pct_of_bf16_peak": 100.0 * flops / fg_s / 1e12 / PEAK_BF16_TFLOPS,
            "entry_point": "ra_forward replayed from a HIP graph", "rank": ranks[-1],
        }
        del fg
    if not args.no_allgather:
        # The all-gather form of the same share: every block resident, one
        # launch (bf16 d_k=128), the state in registers.  Context only; the
        # headline value is the ring with side-stream staging above.
        ag = ra.AllGather(share["gq"], share["gq_pos"], share["gk"], share["gv"], share["gk_pos"])
        ag_s = time_call(ag, args.steps, args.warmup)
        result["allgather"] = {
            "value": flops / ag_s / 1e12, "unit": "TFLOP/s", "ms_per_step": ag_s * 1e3,
            "pct_of_bf16_peak": 100.0 * flops / ag_s / 1e12 / PEAK_BF16_TFLOPS,
            "launches_per_step": 1 if fast else case.n_cp, "rank": ranks[-1],
        }
        del ag
    if not args.no_allgather and not args.no_docs and case.causal:
        # The same share under a document mask: the sequence packed from
        # seeded documents of 512 to 32768 tokens (synth.document_starts),
        # each query seeing only the earlier tokens of its own document.
        # FLOPs are those of the pairs visible under that mask.
        starts = synth.document_starts(case.T, case.seed)
        lo = ra.layouts.document_start_of(share["q_pos"], starts)
        doc_pairs = sum(visible_pairs_docs(share["q_pos"], lo, kp) for kp in share["k_pos"])
        doc_flops = 4 * case.d_k * case.h_q * doc_pairs
        agd = ra.AllGather(share["gq"], share["gq_pos"], share["gk"], share["gv"], share["gk_pos"],
                           q_doc_start=torch.from_numpy(lo).to(dev))
        agd_s = time_call(agd, args.steps, args.warmup)
        result["allgather_docs"] = {
            "value": doc_flops / agd_s / 1e12, "unit": "TFLOP/s", "ms_per_step": agd_s * 1e3,
            "pct_of_bf16_peak": 100.0 * doc_flops / agd_s / 1e12 / PEAK_BF16_TFLOPS,
            "documents": int(len(starts)), "visible_flops": doc_flops,
            "entry_point": "ra_forward_allgather_docs", "rank": ranks[-1],
            # nonzero: the launch splits key walks over workgroups (partial
            # states kept here); only tiles of 128 query rows spanning more
            # than ra_docs_split_span() positions from the first row's
            # document start are split
            "workspace_bytes": int(agd.ws.numel()) if agd.ws is not None else 0,
            "long_tiles": long_tiles(share["q_pos"], lo, span=ra.docs_split_span()),
        }
        del agd
    if not args.no_backward and fast:
        print("[bench] backward", file=sys.stderr, flush=True)
        result["backward"] = time_backward(share, fwd, flops, args.steps, args.warmup, ranks[-1])
    if not args.no_cpu_baseline and len(ranks) >= 1:
        out, lse = fwd.out, fwd.lse
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case, share, out, lse, args.cpu_rows)
    if not args.no_side_workloads and fast and args.config == "llama405b_stage_share" \
            and args.rank is None:
        del fwd, share
        ring.pop("last")
        torch.cuda.empty_cache()
        result["side_workloads"] = {}
        for name in SIDE_WORKLOADS:
            print(f"[bench] side workload {name}", file=sys.stderr, flush=True)
            result["side_workloads"][name] = side_workload(name, dev, args.steps, args.warmup,
                                                           args.timing_reps,
                                                           props.multi_processor_count)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

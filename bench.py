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
import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_F32_TFLOPS = 157.3
HBM_GBPS = 8000.0
METRIC = "causal attention TFLOP/s per rank-share and % of bf16 MFMA peak (1 GPU)"


KERNEL_SOURCE = os.path.join(ROOT, "ring_attention_rank_amd", "csrc", "ra_fast.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_step_kernel_fast_llama405b_stage_share.md")


def kernel_source_sha256():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def committed_traffic(workload):
    """HBM bytes per step launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (calibrated on a plain copy), or None when there is no summary for this
    workload or the kernel source changed since it was taken."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    fields = dict(re.findall(r"^- ([a-z_0-9]+): (\S+)$", text, re.M))
    if fields.get("workload") != workload or fields.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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


def long_tiles(q_pos, q_lo, rows=128, span=8192):
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
    its dk/dv kernels on a side stream.  Its algorithmic flops are five GEMMs
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
            "launches_per_step": 2 + n * (5 if split else 4), "rank": rank}


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
    ap.add_argument("--no-allgather", action="store_true",
                    help="skip timing the all-gather form (every block resident, one launch)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay side line")
    ap.add_argument("--no-docs", action="store_true",
                    help="skip the document-masked all-gather side line")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward of the share (bf16, d_k = 128)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's rank share only; multi-GPU runs are not part of "
              "this build (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return

    case = synth.case_by_name(args.config)
    ranks = case.ranks if args.rank is None else (args.rank,)
    dev = torch.device("cuda", 0)
    props = torch.cuda.get_device_properties(dev)

    total_flops = 0
    total_time = 0.0
    step_ms = []
    per_rank = []
    last = None
    for r in ranks:
        share = build_share(case, r, dev)
        fwd = ra.Forward(share["gq"], share["gq_pos"], share["gk"], share["gv"], share["gk_pos"],
                         side=not args.no_side_stream)
        flops = 4 * case.d_k * case.h_q * sum(share["pairs_per_step"])
        for _ in range(args.warmup):
            fwd()
        torch.cuda.synchronize()
        main_stream = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
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
        total_flops += flops * args.steps
        total_time += wall
        per_rank.append({"rank": r, "median_ms": float(np.median(ms)),
                         "tflops_median": flops / (np.median(ms) * 1e-3) / 1e12,
                         "visible_flops": flops, "staged_bytes": fwd.staged.value,
                         "work": fwd.work.tolist()})
        last = (share, fwd, flops)

    ms_per_step = total_time / (args.steps * len(ranks)) * 1e3
    value = total_flops / total_time / 1e12
    peak = PEAK_BF16_TFLOPS if case.dtype == "bf16" else PEAK_F32_TFLOPS
    share, fwd, flops = last
    n_launch = case.n_cp
    avg_launch_ms = float(np.mean(step_ms)) / n_launch
    achieved = flops / n_launch / (avg_launch_ms * 1e-3) / 1e12
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
        "per_rank": per_rank,
        "roofline": {
            "bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "traffic": committed_traffic(case.name),
            "kernel": ("step_kernel_fast (bf16 MFMA 32x32x16)" if case.dtype == "bf16" and case.d_k == 128
                       else "step_kernel (generic)"),
            "avg_launch_ms": avg_launch_ms, "launches_per_step": n_launch,
            "event_median_ms_per_step": float(np.median(step_ms)),
        },
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    if not args.no_graph:
        # The same ring forward captured once in a HIP graph and replayed
        # (ra.ForwardGraph): the same copies, events and launches, submitted
        # as one graph launch.  Context only; the headline is the eager call.
        fg = ra.ForwardGraph(share["gq"], share["gq_pos"], share["gk"], share["gv"],
                             share["gk_pos"])
        for _ in range(args.warmup):
            fg()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fg()
        torch.cuda.synchronize()
        fg_s = (time.perf_counter() - t0) / args.steps
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
        for _ in range(args.warmup):
            ag()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            ag()
        torch.cuda.synchronize()
        ag_s = (time.perf_counter() - t0) / args.steps
        result["allgather"] = {
            "value": flops / ag_s / 1e12, "unit": "TFLOP/s", "ms_per_step": ag_s * 1e3,
            "pct_of_bf16_peak": 100.0 * flops / ag_s / 1e12 / PEAK_BF16_TFLOPS,
            "launches_per_step": 1 if case.dtype == "bf16" and case.d_k == 128 else case.n_cp,
            "rank": ranks[-1],
        }
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
        for _ in range(args.warmup):
            agd()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            agd()
        torch.cuda.synchronize()
        agd_s = (time.perf_counter() - t0) / args.steps
        result["allgather_docs"] = {
            "value": doc_flops / agd_s / 1e12, "unit": "TFLOP/s", "ms_per_step": agd_s * 1e3,
            "pct_of_bf16_peak": 100.0 * doc_flops / agd_s / 1e12 / PEAK_BF16_TFLOPS,
            "documents": int(len(starts)), "visible_flops": doc_flops,
            "entry_point": "ra_forward_allgather_docs", "rank": ranks[-1],
            # nonzero: the launch splits key walks over workgroups (partial
            # states kept here); only tiles of 128 query rows spanning more
            # than 8192 positions from the first row's document start are split
            "workspace_bytes": int(agd.ws.numel()) if agd.ws is not None else 0,
            "long_tiles": long_tiles(share["q_pos"], lo),
        }
    if not args.no_backward and case.dtype == "bf16" and case.d_k == 128:
        result["backward"] = time_backward(share, fwd, flops, args.steps, args.warmup, ranks[-1])
    if not args.no_cpu_baseline and len(ranks) >= 1:
        out, lse = fwd.out, fwd.lse
        result["cpu_baseline"] = cpu_baseline(case, share, out, lse, args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

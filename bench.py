"""Benchmark: one sequence-parallel rank's document-masked attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload zigzag|ring|ulysses|train|tiny]
                    [--no-cpu-baseline]

A step is one pass of the rank's hot path over resident inputs: for the
default 128K zigzag GQA shard (131072-token packed sequence, SP degree 8,
rank 3 holds 16384 query rows, 32 query / 8 KV heads, head_dim 128) that is
the forward of every non-empty ring step plus the exact LSE merges. Plans are
built once, outside the timed region. Prints ONE JSON line.

Throughput counts only allowed (unmasked) query-key pairs: 4 * head_dim FLOP
per pair per query head for the forward. The roofline object prices the
dominant kernel (attn_fwd) against the bf16 dense matrix-core peak, using the
kernel's own launch durations measured with HIP events on its stream.

The CPU baseline times the fp64 oracle (test infrastructure) on a bounded
sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X published dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X published HBM3E bandwidth


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="zigzag", choices=["zigzag", "ring", "ulysses", "train", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before the run, one plain device-to-device copy of this many MiB (a known-size "
                         "reference for HBM byte counters)")
    return ap.parse_args()


def _traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch recorded by rocprofv3 counter runs, if they were
    taken on the current kernel source (its hash is stored with them)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    src = os.path.join(ROOT, "long_context_sequence_doc_amd", "csrc", f"{kernel}.hip")
    if not (os.path.exists(path) and os.path.exists(src)):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, t, budget_s: float = 20.0):
    """The oracle, as it stands, on a bounded sample: one KV head group's query
    heads over every ring step, all local rows of this rank. Rate = the
    sample's allowed-pair FLOP / wall time."""
    from oracle import attention as A
    from oracle import planner as P
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = 1
    group = w.hq // w.hkv
    heads = list(range(group))           # query heads of KV head 0
    q = W.bf16_to_f32(W.local_rows(t.q, w.q_segs)[:, heads]).astype(np.float64)
    k = W.bf16_to_f32(t.k[:, :1]).astype(np.float64)
    v = W.bf16_to_f32(t.v[:, :1]).astype(np.float64)
    gq = w.q_global_rows()
    pairs = 0
    t0 = time.perf_counter()
    steps_done = 0
    for st in w.steps:
        gk = np.concatenate([np.arange(a, b) for a, b, _ in st.kv_segs])
        pl = P.plan(w.cu, w.q_segs, st.kv_segs, 128, 64)
        if pl.n_tiles == 0:
            continue
        A.forward(q, k[gk], v[gk], gq, gk, w.cu, w.scale)
        pairs += pl.useful_pairs
        steps_done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flop = 4.0 * w.d * len(heads) * pairs
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{w.name}: query heads 0-{len(heads) - 1} (KV head 0), all {w.tq} local rows, "
                      f"{steps_done} non-empty ring steps; fp64 NumPy; {dt:.1f} s wall"}


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    import long_context_sequence_doc_amd as sap
    from long_context_sequence_doc_amd.rank import RankForward

    w = W.by_name(a.workload)
    t = W.make_tensors(w)
    t_plan0 = time.perf_counter()
    rf = RankForward(w.cu, w.q_segs, [s.kv_segs for s in w.steps], w.hq, w.hkv, w.d, w.scale)
    plan_s = time.perf_counter() - t_plan0
    q = torch.from_numpy(W.local_rows(t.q, w.q_segs).view(np.int16)).view(torch.bfloat16).cuda()
    k = torch.from_numpy(t.k.view(np.int16)).view(torch.bfloat16).cuda()
    v = torch.from_numpy(t.v.view(np.int16)).view(torch.bfloat16).cuda()
    stream = torch.cuda.current_stream()
    if a.calibration_copy_mib:
        src = torch.empty(a.calibration_copy_mib << 18, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(a.warmup):
        rf.run(q, k, v, q.stride(0), k.stride(0))
    torch.cuda.synchronize()

    # timed region; the forward launches are bracketed by events on their stream
    fwd_events = []
    merge_events = []
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(a.steps):
        for n, i in enumerate(rf.active):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            out_o, out_l = (rf.o, rf.lse) if n == 0 else (rf.o_part, rf.lse_part)
            e0.record(stream)
            sap.sap_attn_fwd(rf.plans[i], q, k, v, q.stride(0), k.stride(0), w.hq, w.hkv, w.d, w.scale,
                             out_o, out_l)
            e1.record(stream)
            fwd_events.append((e0, e1))
            if n > 0:
                m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                m0.record(stream)
                sap.sap_lse_merge(rf.plans[i], rf.o, rf.lse, rf.o_part, rf.lse_part, rf.tq, w.hq, w.d)
                m1.record(stream)
                merge_events.append((m0, m1))
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / a.steps
    fwd_ms = sum(e0.elapsed_time(e1) for e0, e1 in fwd_events)
    merge_ms = sum(e0.elapsed_time(e1) for e0, e1 in merge_events)

    flop = rf.useful_flop
    value = flop / (ms_per_step * 1e-3) / 1e12
    n_fwd = len(fwd_events)
    fwd_avg_ms = fwd_ms / max(n_fwd, 1)
    flop_per_launch = flop * a.steps / max(n_fwd, 1)
    achieved = flop_per_launch / (fwd_avg_ms * 1e-3) / 1e12 if n_fwd else 0.0
    merge_bytes = rf.merge_rows() * (12 * w.d + 12)
    merge_gbs = (merge_bytes * a.steps / (merge_ms * 1e-3) / 1e9) if merge_events else None
    traffic = _traffic_from_profiles("attn_fwd", w.name)

    line = {
        "metric": "Effective TFLOP/s (unmasked pairs only) + % of bf16 MFMA peak, 128K packed",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": w.name,
            "seq_len": w.total,
            "documents": len(w.lengths),
            "q_rows": w.tq,
            "hq": w.hq,
            "hkv": w.hkv,
            "head_dim": w.d,
            "ring_steps": len(w.steps),
            "nonempty_steps": len(rf.active),
            "useful_pairs_per_head": rf.useful_pairs_per_head,
            "useful_flop_per_step": flop,
            "tile": [128, 64],
            "plan_host_s": round(plan_s, 3),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "launches_per_step": n_fwd // a.steps,
            "avg_launch_ms": round(fwd_avg_ms, 4),
        },
        "merge": None if merge_gbs is None else {
            "bound": "hbm", "achieved_gbs": round(merge_gbs, 1), "peak_gbs": PEAK_HBM_GBS,
            "frac": round(merge_gbs / PEAK_HBM_GBS, 4), "bytes_per_step": merge_bytes,
            "avg_launch_ms": round(merge_ms / len(merge_events), 4)},
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, t)
    rf.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark: one sequence-parallel rank's document-masked attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload zigzag|ring|ulysses|train|tiny]
                    [--forward-only] [--no-cpu-baseline]

A step is one pass of the rank's hot path over resident inputs. For the
default 128K zigzag GQA shard (131072-token packed sequence, SP degree 8,
rank 3 holds 16384 query rows, 32 query / 8 KV heads, head_dim 128) the step
of the headline value is that shard's forward: every non-empty ring step
with its exact LSE merge. The same shard's training step -- that forward,
then the recompute backward (row terms once, one accumulate call per
non-empty step) with the final O and LSE -- is timed after it and reported
under "training_step" (skip it with --forward-only). For the 64K training
workload the headline step is forward + backward. Plans are built once,
outside the timed regions. Prints ONE JSON line.

Throughput counts only allowed (unmasked) query-key pairs: 4 * head_dim FLOP
per pair per query head for the forward and 10 * head_dim for the backward
(recompute of Q K^T and dO V^T, then dV, dK, dQ). The roofline object prices
the dominant kernel against the bf16 dense matrix-core peak, using that
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
    ap.add_argument("--workload", default="zigzag", choices=["zigzag", "ring", "ulysses", "ulysses_gqa", "train", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ranks", action="store_true",
                    help="skip the per-rank sweep of the sharded workloads (zigzag / ring vs balanced layout)")
    ap.add_argument("--forward-only", action="store_true",
                    help="skip the training-step (forward + backward) measurement of forward workloads")
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


def cpu_baseline(w, t, forward_only: bool, min_s: float = 10.0, budget_s: float = 30.0):
    """The oracle, as it stands, on a bounded sample of the same workload: for
    KV heads 0, 1, ... (until about min_s of work, or budget_s), the query
    heads of that KV head over this rank's rows, every non-empty ring step
    (forward per step; then, unless forward-only, the oracle forward over all
    KV rows for the final O / LSE, untimed, and the backward per step). Rate =
    the sample's allowed-pair FLOP (4 D forward + 10 D backward per pair and
    query head) / wall time."""
    from oracle import attention as A
    from oracle import planner as P
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = 1
    group = w.hq // w.hkv
    gq = w.q_global_rows()
    plans = []
    for st in w.steps:
        pl = P.plan(w.cu, w.q_segs, st.kv_segs, 128, 64)
        if pl.n_tiles:
            plans.append((np.concatenate([np.arange(a, b) for a, b, _ in st.kv_segs]), pl.useful_pairs))
    flop, timed, kv_heads = 0.0, 0.0, 0
    for g in range(w.hkv):
        heads = list(range(g * group, (g + 1) * group))
        q = W.bf16_to_f32(W.local_rows(t.q, w.q_segs)[:, heads]).astype(np.float64)
        k = W.bf16_to_f32(t.k[:, g:g + 1]).astype(np.float64)
        v = W.bf16_to_f32(t.v[:, g:g + 1]).astype(np.float64)
        t0 = time.perf_counter()
        for gk, pr in plans:
            A.forward(q, k[gk], v[gk], gq, gk, w.cu, w.scale)
            flop += 4.0 * w.d * group * pr
        timed += time.perf_counter() - t0
        if not forward_only:
            do = W.bf16_to_f32(W.local_rows(t.do, w.q_segs)[:, heads]).astype(np.float64)
            o, lse = A.forward(q, k, v, gq, np.arange(w.total), w.cu, w.scale)   # inputs, not timed
            t0 = time.perf_counter()
            for gk, pr in plans:
                A.backward(q, k[gk], v[gk], do, o, lse, gq, gk, w.cu, w.scale)
                flop += 10.0 * w.d * group * pr
            timed += time.perf_counter() - t0
        kv_heads += 1
        if timed >= min_s or timed * (kv_heads + 1) / kv_heads > budget_s:
            break
    what = "forward per step" if forward_only else \
        "forward per step, then the backward per step from the oracle's final O/LSE (computed untimed)"
    return {"value": flop / timed / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{w.name}: KV heads 0-{kv_heads - 1} with their {group * kv_heads} query heads, all "
                      f"{w.tq} local rows, {len(plans)} non-empty ring steps ({what}); fp64 NumPy; "
                      f"{timed:.1f} s timed"}


class _Timer:
    """HIP events bracketing launches on one stream, grouped by kernel."""

    def __init__(self, stream):
        import torch
        self.torch, self.stream, self.ev = torch, stream, {}

    def run(self, name, fn):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        fn()
        e1.record(self.stream)
        self.ev.setdefault(name, []).append((e0, e1))

    def ms(self, name):
        return sum(a.elapsed_time(b) for a, b in self.ev.get(name, []))

    def count(self, name):
        return len(self.ev.get(name, []))


BALANCE_CHUNK = 1024   # rows per chunk of the document-aware balanced layout


def rank_sweep(w, t, a, stream):
    """Every rank of the sequence-parallel layout ``w`` comes from (its own
    zigzag or contiguous-ring layout) and of the document-aware balanced
    layout from sap_balance, timed one after another on this GPU: per rank and
    ring step, the fused forward (merges in the epilogue). Job time is the
    slowest rank when each rank fetches the KV it needs without lock-step
    (sum over steps, max over ranks), or the sum over ring steps of the
    slowest rank's step when the ring moves in lock-step. Each rank is also
    timed as one call over all the KV it needs."""
    import torch
    import workloads as W
    import long_context_sequence_doc_amd as sap
    from long_context_sequence_doc_amd.rank import RankForward
    p, chunk = w.extra["p"], w.extra["chunk"]
    if w.name.startswith("zigzag"):
        base = ("zigzag", W.zigzag_owner(p), chunk)
    else:
        base = ("ring", list(range(p)), chunk)
    owner, _ = sap.sap_balance(w.cu, p, BALANCE_CHUNK)
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    k, v = dev(t.k), dev(t.v)
    out = {}
    for tag, own, ch in (base, ("balanced", owner.tolist(), BALANCE_CHUNK)):
        flop, rank_ms, step_ms, fetched, touched, one_ms = [], [], [], [], [], []
        for r in range(p):
            wr = W.owner_rank(w, own, r, ch, tag)
            rf = RankForward(wr.cu, wr.q_segs, [s.kv_segs for s in wr.steps], wr.hq, wr.hkv, wr.d, wr.scale)
            q = dev(W.local_rows(t.q, wr.q_segs))
            qs, ks = q.stride(0), k.stride(0)

            def fwd(tm):
                for n, i in enumerate(rf.active):
                    f = sap.sap_attn_fwd if n == 0 else sap.sap_attn_fwd_merge
                    tm.run(i, lambda: f(rf.plans[i], q, k, v, qs, ks, wr.hq, wr.hkv, wr.d, wr.scale, rf.o, rf.lse))
            warm = _Timer(stream)
            for _ in range(a.warmup):
                fwd(warm)
            torch.cuda.synchronize()
            tm = _Timer(stream)
            for _ in range(a.steps):
                fwd(tm)
            torch.cuda.synchronize()
            per_step = [tm.ms(i) / a.steps if i in rf.active else 0.0 for i in range(p)]
            flop.append(rf.useful_flop)
            step_ms.append(per_step)
            rank_ms.append(sum(per_step))
            fetched.append(sum(e - b for i in rf.active if i > 0 for b, e, _ in wr.steps[i].kv_segs))
            # rows of the remote 64-row KV tiles the plans touch (chunks are whole tiles)
            touched.append(sum(rf.infos[i]["n_touched_kv_tiles"] * 64 for i in rf.active if i > 0))
            rf.close()
            # the same rank as one call over all the KV it needs (no ring steps, no merge)
            rc = RankForward.concatenated(wr.cu, wr.q_segs, [s.kv_segs for s in wr.steps], wr.hq, wr.hkv, wr.d,
                                          wr.scale)

            def one(tm):
                tm.run(0, lambda: sap.sap_attn_fwd(rc.plans[0], q, k, v, qs, ks, wr.hq, wr.hkv, wr.d, wr.scale,
                                                   rc.o, rc.lse))
            for _ in range(a.warmup):
                one(warm)
            torch.cuda.synchronize()
            tm = _Timer(stream)
            for _ in range(a.steps):
                one(tm)
            torch.cuda.synchronize()
            one_ms.append(tm.ms(0) / a.steps)
            rc.close()
            del q
        job = max(rank_ms)
        lockstep = sum(max(step_ms[r][s] for r in range(p)) for s in range(p))
        out[tag] = {
            "chunk_rows": ch,
            "useful_flop": flop,
            "ms": [round(x, 4) for x in rank_ms],
            "tflops": [round(f / (m * 1e-3) / 1e12, 1) for f, m in zip(flop, rank_ms)],
            "work_max_over_mean": round(max(flop) / (sum(flop) / p), 4),
            "job_ms": round(job, 4),
            "job_tflops_per_gpu": round(sum(flop) / (job * 1e-3) / 1e12 / p, 1),
            "lockstep_ring_ms": round(lockstep, 4),
            "lockstep_ring_tflops_per_gpu": round(sum(flop) / (lockstep * 1e-3) / 1e12 / p, 1),
            "remote_kv_rows_fetched": fetched,
            "remote_kv_rows_touched": touched,
            "single_call_ms": [round(x, 4) for x in one_ms],
            "single_call_job_tflops_per_gpu": round(sum(flop) / (max(one_ms) * 1e-3) / 1e12 / p, 1),
        }
    out["note"] = ("each rank's forward (ring steps, fused merges) timed alone on this one GPU; job_ms = slowest "
                   "rank (KV fetched as needed), lockstep_ring_ms = sum over ring steps of the slowest rank's step, "
                   "single_call_ms = the rank as one call over all the KV it needs; remote_kv_rows_fetched counts whole "
                   "remote chunks of non-empty steps, remote_kv_rows_touched only the 64-row KV tiles their plans "
                   "touch; communication not included")
    return out


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    import long_context_sequence_doc_amd as sap
    from long_context_sequence_doc_amd.rank import RankBackward, RankForward

    w = W.by_name(a.workload)
    # the training workload's own step is forward + backward; the others' is
    # the forward with its merges, and their training step is reported beside it
    headline_bwd = w.backward
    with_bwd = headline_bwd or not a.forward_only
    t = W.make_tensors(w, with_do=with_bwd)
    t_plan0 = time.perf_counter()
    kv_steps = [s.kv_segs for s in w.steps]
    # partial buffers are kept for the two-pass (separate merge kernel) reference line
    rf = RankForward(w.cu, w.q_segs, kv_steps, w.hq, w.hkv, w.d, w.scale, fused_merge=False)
    rb = RankBackward(w.cu, w.q_segs, kv_steps, w.hq, w.hkv, w.d, w.scale) if with_bwd else None
    plan_s = time.perf_counter() - t_plan0
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    q = dev(W.local_rows(t.q, w.q_segs))
    k, v = dev(t.k), dev(t.v)
    if with_bwd:
        dout = dev(W.local_rows(t.do, w.q_segs))
        # gradient buffers are zeroed once; the timed steps keep accumulating into them
        dq = torch.zeros((rf.tq, w.hq, w.d), dtype=torch.float32, device="cuda")
        dk = torch.zeros((k.shape[0], w.hkv, w.d), dtype=torch.float32, device="cuda")
        dv = torch.zeros_like(dk)
    stream = torch.cuda.current_stream()
    if a.calibration_copy_mib:
        src = torch.empty(a.calibration_copy_mib << 18, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    qs, ks = q.stride(0), k.stride(0)

    def step(tm, backward, fused=True):
        for n, i in enumerate(rf.active):
            if n == 0:
                tm.run("attn_fwd", lambda: sap.sap_attn_fwd(rf.plans[i], q, k, v, qs, ks, w.hq, w.hkv, w.d,
                                                            w.scale, rf.o, rf.lse))
            elif fused:
                # this step's partial merged into the running O / LSE in the kernel epilogue
                tm.run("attn_fwd", lambda: sap.sap_attn_fwd_merge(rf.plans[i], q, k, v, qs, ks, w.hq, w.hkv, w.d,
                                                                  w.scale, rf.o, rf.lse))
            else:
                tm.run("attn_fwd", lambda: sap.sap_attn_fwd(rf.plans[i], q, k, v, qs, ks, w.hq, w.hkv, w.d,
                                                            w.scale, rf.o_part, rf.lse_part))
                tm.run("lse_merge", lambda: sap.sap_lse_merge(rf.plans[i], rf.o, rf.lse, rf.o_part, rf.lse_part,
                                                              rf.tq, w.hq, w.d))
        if backward:
            tm.run("bwd_rowterm", lambda: rb.rowterm(rf.o, dout, qs))
            for i in rb.active:
                tm.run("attn_bwd", lambda: rb.accumulate(i, q, k, v, rf.lse, dout, qs, ks, dq, dk, dv))

    def timed(backward, fused=True):
        warm = _Timer(stream)
        for _ in range(a.warmup):
            step(warm, backward, fused)
        torch.cuda.synchronize()
        tm = _Timer(stream)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(a.steps):
            step(tm, backward, fused)
        end.record(stream)
        torch.cuda.synchronize()
        return tm, start.elapsed_time(end) / a.steps

    fwd_flop = rf.useful_flop
    bwd_flop = rb.useful_flop if rb is not None else 0.0

    def kernel_stats(tm, name, flop_per_step):
        n = tm.count(name)
        if not n:
            return None
        ms = tm.ms(name)
        ach = flop_per_step * a.steps / (ms * 1e-3) / 1e12
        return {"launches_per_step": n // a.steps, "avg_launch_ms": round(ms / n, 4),
                "ms_per_step": round(ms / a.steps, 4), "tflops": round(ach, 3),
                "frac": round(ach / PEAK_BF16_TFLOPS, 4)}

    def hbm_stats(tm, name, bytes_per_step):
        if not tm.count(name):
            return None
        gbs = bytes_per_step * a.steps / (tm.ms(name) * 1e-3) / 1e9
        return {"bound": "hbm", "achieved_gbs": round(gbs, 1), "peak_gbs": PEAK_HBM_GBS,
                "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_step": bytes_per_step,
                "avg_launch_ms": round(tm.ms(name) / tm.count(name), 4)}

    merge_bytes = rf.merge_rows() * (12 * w.d + 12)     # O_acc, O_part read, O_acc written; 3 LSE words
    rowterm_bytes = rf.tq * w.hq * (6 * w.d + 4)         # dO (bf16) and O (fp32) read, D written

    def report(tm, ms_per_step, backward):
        flop = fwd_flop + (bwd_flop if backward else 0.0)
        kernels = {"attn_fwd": kernel_stats(tm, "attn_fwd", fwd_flop),
                   "attn_bwd": kernel_stats(tm, "attn_bwd", bwd_flop) if backward else None,
                   "lse_merge": hbm_stats(tm, "lse_merge", merge_bytes),
                   "bwd_rowterm": hbm_stats(tm, "bwd_rowterm", rowterm_bytes) if backward else None}
        return flop, flop / (ms_per_step * 1e-3) / 1e12, kernels

    tm_h, ms_h = timed(headline_bwd)
    flop, value, kernels = report(tm_h, ms_h, headline_bwd)
    dom_name = "attn_fwd"
    if kernels["attn_bwd"] is not None and kernels["attn_bwd"]["ms_per_step"] > kernels["attn_fwd"]["ms_per_step"]:
        dom_name = "attn_bwd"
    dom = kernels[dom_name]

    line = {
        "metric": "Effective TFLOP/s (unmasked pairs only) + % of bf16 MFMA peak, 128K packed",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_h, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": w.name,
            "step": ("forward (ring steps, LSE merge in the kernel epilogue)" + (" + recompute backward" if headline_bwd
                                                                                 else "")),
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
            "flop_per_pair_per_head": (14 if headline_bwd else 4) * w.d,
            "tiles": {"forward": [rf.block_m, 64], "backward": [64, 128]},
            "plan_host_s": round(plan_s, 3),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": dom_name,
            "achieved": dom["tflops"],
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": dom["frac"],
            "traffic": _traffic_from_profiles(dom_name, w.name),
            "launches_per_step": dom["launches_per_step"],
            "avg_launch_ms": dom["avg_launch_ms"],
        },
        "kernels": kernels,
    }
    if len(rf.active) > 1 and not headline_bwd:
        # the headline step's launches one by one: each non-empty ring step's
        # useful FLOP, time and rate (step 0 writes, later steps merge)
        def by_step(tm):
            for n, i in enumerate(rf.active):
                f = sap.sap_attn_fwd if n == 0 else sap.sap_attn_fwd_merge
                tm.run(i, lambda: f(rf.plans[i], q, k, v, qs, ks, w.hq, w.hkv, w.d, w.scale, rf.o, rf.lse))
        warm = _Timer(stream)
        for _ in range(a.warmup):
            by_step(warm)
        torch.cuda.synchronize()
        tm_s = _Timer(stream)
        for _ in range(a.steps):
            by_step(tm_s)
        torch.cuda.synchronize()
        line["ring_steps"] = []
        for i in rf.active:
            inf = rf.infos[i]
            f_i = inf["useful_pairs_per_head"] * w.hq * 4 * w.d
            ms_i = tm_s.ms(i) / a.steps
            line["ring_steps"].append({"step": i, "touched_q_tiles": inf["n_touched_q_tiles"], "tiles": inf["n_tiles"],
                                       "useful_flop": f_i, "ms": round(ms_i, 4),
                                       "tflops": round(f_i / (ms_i * 1e-3) / 1e12, 1)})
        # the same forward as one call over all steps' KV (a rank holding every chunk)
        rc = RankForward.concatenated(w.cu, w.q_segs, kv_steps, w.hq, w.hkv, w.d, w.scale)
        rc_plan = rc.plans[0]

        def one_call(tm):
            tm.run("attn_fwd", lambda: sap.sap_attn_fwd(rc_plan, q, k, v, qs, ks, w.hq, w.hkv, w.d, w.scale,
                                                        rc.o, rc.lse))
        warm = _Timer(stream)
        for _ in range(a.warmup):
            one_call(warm)
        torch.cuda.synchronize()
        tm_c = _Timer(stream)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(a.steps):
            one_call(tm_c)
        end.record(stream)
        torch.cuda.synchronize()
        ms_c = start.elapsed_time(end) / a.steps
        line["forward_single_call"] = {
            "step": "forward as one call over every step's KV segments (all chunks resident; no merge)",
            "value": round(fwd_flop / (ms_c * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "ms_per_step": round(ms_c, 4),
            "kernels": {"attn_fwd": kernel_stats(tm_c, "attn_fwd", fwd_flop)}}
        rc.close()
        # two calls: the rank's own chunks, then every remote chunk at once (merged)
        rr = RankForward.local_then_remote(w.cu, w.q_segs, kv_steps, w.hq, w.hkv, w.d, w.scale)

        def two_calls(tm):
            tm.run("attn_fwd", lambda: sap.sap_attn_fwd(rr.plans[0], q, k, v, qs, ks, w.hq, w.hkv, w.d, w.scale,
                                                        rr.o, rr.lse))
            tm.run("attn_fwd", lambda: sap.sap_attn_fwd_merge(rr.plans[1], q, k, v, qs, ks, w.hq, w.hkv, w.d,
                                                              w.scale, rr.o, rr.lse))
        warm = _Timer(stream)
        for _ in range(a.warmup):
            two_calls(warm)
        torch.cuda.synchronize()
        tm_r = _Timer(stream)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(a.steps):
            two_calls(tm_r)
        end.record(stream)
        torch.cuda.synchronize()
        ms_r = start.elapsed_time(end) / a.steps
        line["forward_local_then_remote"] = {
            "step": "forward as two calls: the rank's own chunks, then all remote chunks at once (merge in the "
                    "epilogue)",
            "value": round(fwd_flop / (ms_r * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "ms_per_step": round(ms_r, 4),
            "kernels": {"attn_fwd": kernel_stats(tm_r, "attn_fwd", fwd_flop)}}
        rr.close()
        # reference: the same forward with a separate merge pass per step
        tm_2, ms_2 = timed(False, fused=False)
        _, value_2, kernels_2 = report(tm_2, ms_2, False)
        line["forward_two_pass"] = {"step": "forward (ring steps + separate lse_merge pass per step)",
                                    "value": round(value_2, 3), "unit": "TFLOP/s", "ms_per_step": round(ms_2, 4),
                                    "kernels": kernels_2}
    if with_bwd and not headline_bwd and len(rf.active) > 1:
        # the same training step as one forward call and one backward call over
        # every step's KV (a rank holding every chunk)
        rc = RankForward.concatenated(w.cu, w.q_segs, kv_steps, w.hq, w.hkv, w.d, w.scale)
        rbc = RankBackward.concatenated(w.cu, w.q_segs, kv_steps, w.hq, w.hkv, w.d, w.scale)

        def one_train(tm):
            tm.run("attn_fwd", lambda: sap.sap_attn_fwd(rc.plans[0], q, k, v, qs, ks, w.hq, w.hkv, w.d, w.scale,
                                                        rc.o, rc.lse))
            tm.run("bwd_rowterm", lambda: rbc.rowterm(rc.o, dout, qs))
            tm.run("attn_bwd", lambda: rbc.accumulate(0, q, k, v, rc.lse, dout, qs, ks, dq, dk, dv))
        warm = _Timer(stream)
        for _ in range(a.warmup):
            one_train(warm)
        torch.cuda.synchronize()
        tm_c = _Timer(stream)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(a.steps):
            one_train(tm_c)
        end.record(stream)
        torch.cuda.synchronize()
        ms_c = start.elapsed_time(end) / a.steps
        line["training_step_single_call"] = {
            "step": "forward + backward as one call each over every step's KV segments (all chunks resident)",
            "value": round((fwd_flop + bwd_flop) / (ms_c * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "ms_per_step": round(ms_c, 4),
            "kernels": {"attn_fwd": kernel_stats(tm_c, "attn_fwd", fwd_flop),
                        "attn_bwd": kernel_stats(tm_c, "attn_bwd", bwd_flop)}}
        rc.close()
        rbc.close()
        # the same training step as two calls each: own chunks, then all remote chunks at once
        rr = RankForward.local_then_remote(w.cu, w.q_segs, kv_steps, w.hq, w.hkv, w.d, w.scale)
        rbr = RankBackward.local_then_remote(w.cu, w.q_segs, kv_steps, w.hq, w.hkv, w.d, w.scale)

        def two_train(tm):
            tm.run("attn_fwd", lambda: sap.sap_attn_fwd(rr.plans[0], q, k, v, qs, ks, w.hq, w.hkv, w.d, w.scale,
                                                        rr.o, rr.lse))
            tm.run("attn_fwd", lambda: sap.sap_attn_fwd_merge(rr.plans[1], q, k, v, qs, ks, w.hq, w.hkv, w.d,
                                                              w.scale, rr.o, rr.lse))
            tm.run("bwd_rowterm", lambda: rbr.rowterm(rr.o, dout, qs))
            for i in rbr.active:
                tm.run("attn_bwd", lambda: rbr.accumulate(i, q, k, v, rr.lse, dout, qs, ks, dq, dk, dv))
        warm = _Timer(stream)
        for _ in range(a.warmup):
            two_train(warm)
        torch.cuda.synchronize()
        tm_c = _Timer(stream)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(a.steps):
            two_train(tm_c)
        end.record(stream)
        torch.cuda.synchronize()
        ms_c = start.elapsed_time(end) / a.steps
        line["training_step_local_then_remote"] = {
            "step": "forward + backward as two calls each: the rank's own chunks, then all remote chunks at once",
            "value": round((fwd_flop + bwd_flop) / (ms_c * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "ms_per_step": round(ms_c, 4),
            "kernels": {"attn_fwd": kernel_stats(tm_c, "attn_fwd", fwd_flop),
                        "attn_bwd": kernel_stats(tm_c, "attn_bwd", bwd_flop)}}
        rr.close()
        rbr.close()
    if with_bwd and not headline_bwd:
        # the same shard's training step: forward + recompute backward
        tm_t, ms_t = timed(True)
        tflop, tvalue, tkernels = report(tm_t, ms_t, True)
        line["training_step"] = {"step": "forward (ring steps, fused merges) + recompute backward",
                                 "value": round(tvalue, 3), "unit": "TFLOP/s",
                                 "pct_of_peak": round(100.0 * tvalue / PEAK_BF16_TFLOPS, 2),
                                 "ms_per_step": round(ms_t, 4), "useful_flop_per_step": tflop,
                                 "flop_per_pair_per_head": 14 * w.d, "kernels": tkernels}
    if not a.no_ranks and not a.forward_only and "p" in w.extra and "chunk" in w.extra:
        line["ranks"] = rank_sweep(w, t, a, stream)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, t, not headline_bwd)
    rf.close()
    if rb is not None:
        rb.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

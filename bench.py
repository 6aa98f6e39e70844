"""Benchmark: one sequence-parallel rank's document-masked attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload zigzag|ring|ulysses|ulysses_gqa|train|tiny]
                    [--forward-only] [--no-cpu-baseline] [--no-ranks] [--no-workloads]

A step is one pass of the rank's hot path over resident inputs. For the
default 128K zigzag GQA shard (131072-token packed sequence, SP degree 8,
rank 3 holds 16384 query rows, 32 query / 8 KV heads, head_dim 128) the step
of the headline value is that shard's forward: every non-empty ring step
with its exact LSE merge (folded into the forward kernel's epilogue). The same
shard's training step -- that forward, then the recompute backward (row terms
once, then per non-empty step the dK / dV pass and the dQ pass) with the final
O and LSE -- is timed after it and reported under "training_step" (skip it
with --forward-only). The other workloads of the measurement plan (the 32K
ring rank, the 512K Ulysses shard with both head splits, the 64K training
shard's forward + backward) are timed after it under "workloads" (skip with
--no-workloads). For the 64K training workload as --workload the headline step
is forward + backward. Plans are built once, outside the timed regions.
Prints ONE JSON line.

Throughput counts only allowed (unmasked) query-key pairs: 4 * head_dim FLOP
per pair per query head for the forward and 10 * head_dim for the backward
(recompute of Q K^T and dO V^T, then dV, dK, dQ). Per kernel, the dK / dV
pass is credited with its own four products (8 * head_dim: S, dP, dV, dK) and
the dQ pass with its three (6 * head_dim: S and dP recomputed, dQ). Each
kernel's rate comes from its own launch durations, measured with HIP events
on the stream it is launched on, and is priced against the bf16 dense
matrix-core peak.

The CPU baseline times the fp64 oracle (test infrastructure) on the same
workload on this host's cores: a process pool of one worker per core (at most
16), one BLAS thread each, over (query head, ring step, document, block of
query rows) units.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X published dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X published HBM3E bandwidth
BALANCE_CHUNK = 1024        # rows per chunk of the document-aware balanced layout
# FLOP per allowed (query, key) pair per query head, in units of head_dim
FWD_PER_D, BWD_PER_D, BWD_KV_PER_D, BWD_DQ_PER_D = 4, 10, 8, 6
KERNEL_SOURCE = {"attn_fwd": "attn_fwd.hip", "attn_bwd_kv": "attn_bwd.hip", "attn_bwd_dq": "attn_bwd.hip"}


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--counters-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn the counter files of two rocprofv3 --pmc runs (FETCH_SIZE, then "
                         "WRITE_SIZE) of 'bench.py --steps 3 --warmup 1 --no-ranks --no-workloads --no-cpu-baseline "
                         "--calibration-copy-mib 1024' into profiles/<kernel>_<workload>_traffic.json records")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="zigzag", choices=["zigzag", "ring", "ulysses", "ulysses_gqa", "train", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ranks", action="store_true",
                    help="skip the per-rank sweep of the sharded workloads (zigzag / ring vs balanced layout)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads (32K ring, 512K Ulysses, 64K training shard)")
    ap.add_argument("--forward-only", action="store_true",
                    help="skip the training-step (forward + backward) measurement of forward workloads")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before the run, one plain device-to-device copy of this many MiB (a known-size "
                         "reference for HBM byte counters)")
    return ap.parse_args()


def _sources_sha256(kernel: str):
    """Hash of what decides a kernel's HBM traffic: its source, the shared
    global -> LDS copy header and the host planner (tile lists, work order and
    chunking); None if a file is missing."""
    csrc = os.path.join(ROOT, "long_context_sequence_doc_amd", "csrc")
    h = hashlib.sha256()
    for name in (KERNEL_SOURCE.get(kernel, kernel + ".hip"), "lds_copy.h", "planner.cpp"):
        path = os.path.join(csrc, name)
        if not os.path.exists(path):
            return None
        h.update(open(path, "rb").read())
    return h.hexdigest()


def _traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch recorded by rocprofv3 counter runs, if they were
    taken on the current kernel source and planner (their hash is stored with
    them)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = _sources_sha256(kernel)
    if sha is None or rec.get("sources_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# HBM traffic records from rocprofv3 counter files

COUNTER_RUN = ("python3 bench.py --steps 3 --warmup 1 --no-ranks --no-workloads --no-cpu-baseline "
               "--calibration-copy-mib 1024")


def _read_counter_csv(path, counter):
    """{dispatch id: (kernel name, value in KiB)} of one rocprofv3 counter file."""
    import csv
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        did = int(r["Dispatch_Id"])
        name, val = r["Kernel_Name"], float(r["Counter_Value"])
        prev = out.get(did, (name, 0.0))[1]
        out[did] = (name, prev + val)          # summed over the counter's instances
    return dict(sorted(out.items()))


def _algorithmic_bytes(w):
    """Bytes each kernel must move per launch at the least (each operand read
    or written once), averaged over the launches of one step of the rank:
    the forward's ring steps (fused merges), the backward's dK / dV and dQ
    passes of each non-empty ring step."""
    import long_context_sequence_doc_amd as sap
    d, hq, hkv = w.d, w.hq, w.hkv
    def rows_of(plan):
        touched, desc = sap.sap_plan_q_tiles(plan)
        return int(desc[touched, 1].sum())
    fwd, kv, dq = [], [], []
    first = True
    for st in w.steps:
        pf = sap.sap_plan(w.cu, w.q_segs, st.kv_segs, 128, 64)
        inf = sap.sap_plan_info(pf)
        if inf["n_tiles"] == 0:
            continue
        qr, kr = rows_of(pf), inf["n_touched_kv_tiles"] * 64
        o_bytes = qr * hq * (4 * d + 4) * (1 if first else 2)      # O + LSE written (merging steps also read)
        fwd.append(qr * hq * d * 2 + kr * hkv * d * 2 * 2 + o_bytes)
        pb = sap.sap_plan(w.cu, w.q_segs, st.kv_segs, 64, 128)
        ib = sap.sap_plan_info(pb)
        qb, kb = rows_of(pb), ib["n_touched_kv_tiles"] * 128
        reads = qb * hq * d * 2 * 2 + kb * hkv * d * 2 * 2 + qb * hq * 4 * 2     # Q, dO, K, V, LSE, D
        kv.append(reads + kb * hkv * d * 4 * 2 * 2)                              # dK, dV read and written
        dq.append(reads + qb * hq * d * 4 * 2)                                   # dQ read and written
        first = False
    avg = lambda x: int(round(sum(x) / len(x)))
    return {"attn_fwd": avg(fwd), "attn_bwd_kv": avg(kv), "attn_bwd_dq": avg(dq)}, len(fwd)


def counters_summary(fetch_csv, write_csv, workload="zigzag", warmup=1, steps=3, calib_mib=1024):
    """HBM bytes per launch of the forward and the two backward passes from
    FETCH_SIZE / WRITE_SIZE counter runs of COUNTER_RUN, scaled by what the
    same counters read for the run's plain calibration copy of calib_mib MiB
    (a copy that reads and writes calib_mib MiB), written to
    profiles/<kernel>_<workload>_traffic.json with the hash of the kernel's
    source. The forward's launches are the first ones of the run (the
    headline step: warm-up and timed steps, one launch per non-empty ring
    step); the backward's are the last ones (the training step as ring
    steps, run last)."""
    import workloads as W
    w = W.by_name(workload)
    fetch = _read_counter_csv(fetch_csv, "FETCH_SIZE")
    write = _read_counter_csv(write_csv, "WRITE_SIZE")
    kib = calib_mib * 1024.0
    def calib(table):
        vals = [v for n, v in table.values() if "copyBuffer" in n and v > 0.25 * kib]
        if not vals:
            raise SystemExit("no calibration copy in the counter file (run with --calibration-copy-mib)")
        return vals[0]
    fs, ws = kib / calib(fetch), kib / calib(write)
    alg, n_steps = _algorithmic_bytes(w)
    per_phase = (warmup + steps) * n_steps
    out = []
    for key, pattern, src, which in (("attn_fwd", "attn_fwd_kernel", "attn_fwd.hip", "first"),
                                     ("attn_bwd_kv", "attn_bwd_kv_kernel", "attn_bwd.hip", "last"),
                                     ("attn_bwd_dq", "attn_bwd_dq_kernel", "attn_bwd.hip", "last")):
        fv = [v for n, v in fetch.values() if pattern in n]
        wv = [v for n, v in write.values() if pattern in n]
        if len(fv) < per_phase or len(wv) < per_phase:
            raise SystemExit(f"{key}: {len(fv)} / {len(wv)} dispatches, expected at least {per_phase}")
        fv = fv[:per_phase] if which == "first" else fv[-per_phase:]
        wv = wv[:per_phase] if which == "first" else wv[-per_phase:]
        by_step_f = [sum(fv[i::n_steps]) / (warmup + steps) for i in range(n_steps)]
        by_step_w = [sum(wv[i::n_steps]) / (warmup + steps) for i in range(n_steps)]
        bpl = (sum(fv) / per_phase * fs + sum(wv) / per_phase * ws) * 1024.0
        rec = {
            "kernel": key, "workload": w.name,
            "what": f"HBM bytes per {key} launch, averaged over the {n_steps} non-empty ring-step launches of one step "
                    f"({'the headline forward, merges in the epilogue' if key == 'attn_fwd' else 'the training step backward'})",
            "commands": [f"cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <repo>/gpurun_out/pmc/fetch "
                         f"-o fetch -- {COUNTER_RUN.replace('bench.py', '<repo>/bench.py')}",
                         f"cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <repo>/gpurun_out/pmc/write "
                         f"-o write -- {COUNTER_RUN.replace('bench.py', '<repo>/bench.py')}",
                         "python3 bench.py --counters-summary <fetch csv> <write csv>"],
            "calibration": {"kernel": f"__amd_rocclr_copyBuffer (a plain copy of {calib_mib} MiB)", "true_kib_read": kib,
                            "true_kib_written": kib, "FETCH_SIZE_kib": calib(fetch), "WRITE_SIZE_kib": calib(write),
                            "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)},
            "raw_kib_per_launch_by_ring_step": {"FETCH_SIZE": [round(x, 1) for x in by_step_f],
                                                "WRITE_SIZE": [round(x, 1) for x in by_step_w]},
            "dispatches_used": f"the {which} {per_phase} {pattern} dispatches of the run",
            "bytes_per_launch": int(round(bpl)),
            "algorithmic_bytes_per_launch": alg[key],
            "traffic_over_algorithmic": round(bpl / alg[key], 3),
            "sources": [f"long_context_sequence_doc_amd/csrc/{src}", "long_context_sequence_doc_amd/csrc/lds_copy.h",
                        "long_context_sequence_doc_amd/csrc/planner.cpp"],
            "sources_sha256": _sources_sha256(key),
        }
        path = os.path.join(ROOT, "profiles", f"{key}_{w.name}_traffic.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        out.append((path, rec["bytes_per_launch"], alg[key]))
    for path, b, a in out:
        print(f"{path}: {b / 1e6:.1f} MB per launch, algorithmic {a / 1e6:.1f} MB ({b / a:.2f}x)")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle over a process pool

_POOL_DATA = {}


def _pool_init(paths, cu, scale):
    """Worker set-up (a fresh interpreter: the pool is spawned, nothing of the
    GPU process is inherited): one BLAS thread, the inputs mapped read-only."""
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:
        pass
    for key, p in paths.items():
        _POOL_DATA[key] = np.load(p, mmap_mode="r")
    _POOL_DATA["cu"] = cu
    _POOL_DATA["scale"] = scale


def _pool_unit(unit):
    """One (query head, KV head, query rows, key rows) unit of the oracle's
    forward; returns its wall time."""
    from oracle import attention as A
    h, g, rows, cols = unit
    f64 = lambda bits: (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    d = _POOL_DATA
    t0 = time.perf_counter()
    A.forward(f64(d["q"][rows, h:h + 1]), f64(d["k"][cols, g:g + 1]), f64(d["v"][cols, g:g + 1]),
              d["gq"][rows], d["gk"][cols], d["cu"], d["scale"])
    return time.perf_counter() - t0


def cpu_baseline(w, t, min_s: float = 10.0, budget_s: float = 30.0):
    """The oracle, as it stands, on the workload's forward (every non-empty
    ring step), spread over a spawned process pool of one worker per core (at
    most 16: a GPU machine's share), one BLAS thread each. Work units are (query
    head, ring step, document, block of <= 1024 query rows): the oracle's own
    forward on those rows against that document's keys in the step. Query
    heads are taken in order, whole KV groups at a time, until about min_s
    seconds of wall time (or all heads). Rate = the sample's allowed-pair FLOP
    (4 D per pair and query head) / wall time of its units."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from oracle import planner as P
    try:
        workers = len(os.sched_getaffinity(0))
    except AttributeError:
        workers = os.cpu_count() or 1
    workers = max(1, min(16, workers))
    group = w.hq // w.hkv
    gq = w.q_global_rows()
    cu = np.asarray(w.cu, dtype=np.int64)
    q_loc = W_local_rows(t.q, w.q_segs)
    steps = []
    for st in w.steps:
        pl = P.plan(w.cu, w.q_segs, st.kv_segs, 128, 64)
        if pl.n_tiles:
            steps.append((np.concatenate([np.arange(a, b) for a, b, _ in st.kv_segs]), pl.useful_pairs))
    doc_q = np.searchsorted(cu, gq, side="right") - 1
    units_of_head = []
    for gk, _ in steps:
        doc_k = np.searchsorted(cu, gk, side="right") - 1
        for dd in np.unique(doc_q):
            rows = np.nonzero(doc_q == dd)[0]
            cols = gk[doc_k == dd]
            if len(cols) == 0:
                continue
            for i in range(0, len(rows), 1024):
                units_of_head.append((rows[i:i + 1024], cols))
    tmp = tempfile.mkdtemp(prefix="sap_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    paths = {}
    try:
        for key, arr in (("q", q_loc), ("k", t.k), ("v", t.v), ("gq", gq), ("gk", np.arange(w.total))):
            paths[key] = os.path.join(tmp, key + ".npy")
            np.save(paths[key], np.ascontiguousarray(arr))
        # a worker that cannot start breaks the pool (an error), it is not respawned
        with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn"), initializer=_pool_init,
                                 initargs=(paths, cu, w.scale)) as pool:
            list(pool.map(abs, range(4 * workers)))         # workers started and their inputs mapped
            flop, wall, heads = 0.0, 0.0, 0
            for g in range(w.hkv):
                units = [(h, g, r, c) for h in range(g * group, (g + 1) * group) for r, c in units_of_head]
                t0 = time.perf_counter()
                list(pool.map(_pool_unit, units, chunksize=1))
                wall += time.perf_counter() - t0
                flop += FWD_PER_D * w.d * group * sum(pr for _, pr in steps)
                heads += group
                if wall >= min_s or wall * (g + 2) / (g + 1) > budget_s:
                    break
    finally:
        for p in paths.values():
            if os.path.exists(p):
                os.remove(p)
        os.rmdir(tmp)
    n_units = len(units_of_head) * heads
    return {"value": flop / wall / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{w.name} forward: query heads 0-{heads - 1} of {w.hq} (KV heads 0-{heads // group - 1}), all "
                      f"{w.tq} local rows, {len(steps)} non-empty ring steps; {n_units} units of (query head, ring "
                      f"step, document, <= 1024 query rows) on a spawned pool of {workers} processes with one BLAS "
                      f"thread each; fp64 NumPy; {wall:.1f} s wall"}


def W_local_rows(bits, segs):
    import workloads as W
    return W.local_rows(bits, segs)


# ---------------------------------------------------------------------------
# GPU timing

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


def _timed(a, stream, body):
    """W untimed steps, then K timed ones bracketed by events on the stream;
    returns the per-kernel timer and ms per step."""
    import torch
    warm = _Timer(stream)
    for _ in range(a.warmup):
        body(warm)
    torch.cuda.synchronize()
    tm = _Timer(stream)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(a.steps):
        body(tm)
    end.record(stream)
    torch.cuda.synchronize()
    return tm, start.elapsed_time(end) / a.steps


def _kernel_stats(a, tm, name, flop_per_step, kernel=None, workload=None, per_d=None):
    n = tm.count(name)
    if not n:
        return None
    ms = tm.ms(name)
    ach = flop_per_step * a.steps / (ms * 1e-3) / 1e12
    out = {"launches_per_step": n // a.steps, "avg_launch_ms": round(ms / n, 4), "ms_per_step": round(ms / a.steps, 4),
           "tflops": round(ach, 3), "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    if per_d is not None:
        out["flop_per_pair_per_head"] = per_d
    if kernel is not None:
        out["traffic"] = _traffic_from_profiles(kernel, workload)
    return out


def _hbm_stats(a, tm, name, bytes_per_step):
    if not tm.count(name):
        return None
    gbs = bytes_per_step * a.steps / (tm.ms(name) * 1e-3) / 1e9
    return {"bound": "hbm", "achieved_gbs": round(gbs, 1), "peak_gbs": PEAK_HBM_GBS,
            "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_step": bytes_per_step,
            "avg_launch_ms": round(tm.ms(name) / tm.count(name), 4)}


class _Rank:
    """A workload's rank on the GPU: inputs, forward / backward runners and
    the launches of one step, each named by its kernel."""

    def __init__(self, w, t, with_bwd, form="ring"):
        import torch
        from long_context_sequence_doc_amd.rank import RankBackward, RankForward
        self.w = w
        kv = [s.kv_segs for s in w.steps]
        if form == "ring":
            self.rf = RankForward(w.cu, w.q_segs, kv, w.hq, w.hkv, w.d, w.scale, fused_merge=False)
            self.rb = RankBackward(w.cu, w.q_segs, kv, w.hq, w.hkv, w.d, w.scale) if with_bwd else None
        elif form == "one":
            self.rf = RankForward.concatenated(w.cu, w.q_segs, kv, w.hq, w.hkv, w.d, w.scale)
            self.rb = RankBackward.concatenated(w.cu, w.q_segs, kv, w.hq, w.hkv, w.d, w.scale) if with_bwd else None
        else:
            self.rf = RankForward.local_then_remote(w.cu, w.q_segs, kv, w.hq, w.hkv, w.d, w.scale)
            self.rb = RankBackward.local_then_remote(w.cu, w.q_segs, kv, w.hq, w.hkv, w.d, w.scale) if with_bwd \
                else None
        dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
        self.q = dev(W_local_rows(t.q, w.q_segs))
        self.k, self.v = dev(t.k), dev(t.v)
        self.qs, self.ks = self.q.stride(0), self.k.stride(0)
        if with_bwd:
            self.dout = dev(W_local_rows(t.do, w.q_segs))
            # gradient buffers are zeroed once; the timed steps keep accumulating into them
            self.dq = torch.zeros((self.rf.tq, w.hq, w.d), dtype=torch.float32, device="cuda")
            self.dk = torch.zeros((self.k.shape[0], w.hkv, w.d), dtype=torch.float32, device="cuda")
            self.dv = torch.zeros_like(self.dk)

    @property
    def pairs(self):
        return self.rf.useful_pairs_per_head * self.w.hq

    def forward(self, tm, fused=True):
        import long_context_sequence_doc_amd as sap
        rf, w = self.rf, self.w
        for n, i in enumerate(rf.active):
            args = (rf.plans[i], self.q, self.k, self.v, self.qs, self.ks, w.hq, w.hkv, w.d, w.scale)
            if n == 0:
                tm.run("attn_fwd", lambda: sap.sap_attn_fwd(*args, rf.o, rf.lse))
            elif fused:
                # this step's partial merged into the running O / LSE in the kernel epilogue
                tm.run("attn_fwd", lambda: sap.sap_attn_fwd_merge(*args, rf.o, rf.lse))
            else:
                tm.run("attn_fwd", lambda: sap.sap_attn_fwd(*args, rf.o_part, rf.lse_part))
                tm.run("lse_merge", lambda: sap.sap_lse_merge(rf.plans[i], rf.o, rf.lse, rf.o_part, rf.lse_part,
                                                              rf.tq, w.hq, w.d))

    def backward(self, tm):
        rb, rf = self.rb, self.rf
        tm.run("bwd_rowterm", lambda: rb.rowterm(rf.o, self.dout, self.qs))
        for i in rb.active:
            tm.run("attn_bwd_kv", lambda: rb.dkdv(i, self.q, self.k, self.v, rf.lse, self.dout, self.qs, self.ks,
                                                  self.dk, self.dv))
            tm.run("attn_bwd_dq", lambda: rb.dq(i, self.q, self.k, self.v, rf.lse, self.dout, self.qs, self.ks,
                                                self.dq))

    def step(self, tm, backward, fused=True):
        self.forward(tm, fused)
        if backward:
            self.backward(tm)

    def report(self, a, tm, ms, backward, label):
        """The step's value and every kernel's own rate."""
        w = self.w
        fwd = FWD_PER_D * w.d * self.pairs
        bwd = BWD_PER_D * w.d * self.pairs if backward else 0.0
        kernels = {"attn_fwd": _kernel_stats(a, tm, "attn_fwd", fwd, "attn_fwd", w.name, FWD_PER_D * w.d)}
        if tm.count("lse_merge"):
            kernels["lse_merge"] = _hbm_stats(a, tm, "lse_merge", self.rf.merge_rows() * (12 * w.d + 12))
        if backward:
            kv = _kernel_stats(a, tm, "attn_bwd_kv", BWD_KV_PER_D * w.d * self.pairs, "attn_bwd_kv", w.name,
                               BWD_KV_PER_D * w.d)
            dq = _kernel_stats(a, tm, "attn_bwd_dq", BWD_DQ_PER_D * w.d * self.pairs, "attn_bwd_dq", w.name,
                               BWD_DQ_PER_D * w.d)
            bwd_ms = (tm.ms("attn_bwd_kv") + tm.ms("attn_bwd_dq")) / a.steps
            ach = bwd / (bwd_ms * 1e-3) / 1e12
            kernels["attn_bwd"] = {"useful_tflops": round(ach, 3), "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                                   "ms_per_step": round(bwd_ms, 4), "flop_per_pair_per_head": BWD_PER_D * w.d,
                                   "note": "dK/dV pass + dQ pass, useful FLOP (10 D per pair; they execute 14 D)"}
            kernels["attn_bwd_kv"] = kv
            kernels["attn_bwd_dq"] = dq
            kernels["bwd_rowterm"] = _hbm_stats(a, tm, "bwd_rowterm", self.rf.tq * w.hq * (6 * w.d + 4))
        value = (fwd + bwd) / (ms * 1e-3) / 1e12
        return {"step": label, "value": round(value, 3), "unit": "TFLOP/s",
                "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2), "ms_per_step": round(ms, 4),
                "useful_flop_per_step": fwd + bwd,
                "flop_per_pair_per_head": (FWD_PER_D + (BWD_PER_D if backward else 0)) * w.d, "kernels": kernels}

    def close(self):
        self.rf.close()
        if self.rb is not None:
            self.rb.close()


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
            tm, _ = _timed(a, stream, fwd)
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
            tm, _ = _timed(a, stream, lambda tm: tm.run(0, lambda: sap.sap_attn_fwd(
                rc.plans[0], q, k, v, qs, ks, wr.hq, wr.hkv, wr.d, wr.scale, rc.o, rc.lse)))
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


def other_workloads(a, stream, skip):
    """The measurement plan's other workloads, each as its rank's step on this
    GPU: the 32K ring rank 3 (32 heads; ring steps with fused merges), the
    512K Ulysses shard (4 heads; and its GQA-aware split, 4 query heads / 1 KV
    head), both one full-sequence call, and the 64K training shard (5 heads,
    forward + backward)."""
    import torch
    import workloads as W
    out = {}
    for name, backward in (("ring", False), ("ulysses", False), ("ulysses_gqa", False), ("train", True)):
        if name == skip:
            continue
        w = W.by_name(name)
        t = W.make_tensors(w, with_do=backward)
        r = _Rank(w, t, backward)
        tm, ms = _timed(a, stream, lambda tm: r.step(tm, backward))
        rep = r.report(a, tm, ms, backward, "forward + recompute backward" if backward else
                       ("forward (ring steps, LSE merge in the kernel epilogue)" if len(r.rf.active) > 1 else
                        "forward (one full-sequence call)"))
        rep["config"] = {"workload": w.name, "seq_len": w.total, "documents": len(w.lengths), "q_rows": w.tq,
                         "hq": w.hq, "hkv": w.hkv, "head_dim": w.d, "ring_steps": len(w.steps),
                         "nonempty_steps": len(r.rf.active), "useful_pairs_per_head": r.rf.useful_pairs_per_head,
                         "tiles": {"forward": [r.rf.block_m, 64], "backward": [64, 128]}}
        out[name] = rep
        r.close()
        del r, t
        torch.cuda.empty_cache()
    return out


def main():
    a = _args()
    if a.counters_summary:
        counters_summary(*a.counters_summary, workload=a.workload)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}): every run here uses a single MI355X; "
              f"run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    import long_context_sequence_doc_amd as sap
    from long_context_sequence_doc_amd.rank import RankForward

    w = W.by_name(a.workload)
    # the training workload's own step is forward + backward; the others' is
    # the forward with its merges, and their training step is reported beside it
    headline_bwd = w.backward
    with_bwd = headline_bwd or not a.forward_only
    t = W.make_tensors(w, with_do=with_bwd)
    t_plan0 = time.perf_counter()
    r = _Rank(w, t, with_bwd)
    plan_s = time.perf_counter() - t_plan0
    rf = r.rf
    stream = torch.cuda.current_stream()
    if a.calibration_copy_mib:
        src = torch.empty(a.calibration_copy_mib << 18, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    tm_h, ms_h = _timed(a, stream, lambda tm: r.step(tm, headline_bwd))
    head = r.report(a, tm_h, ms_h, headline_bwd, "")
    kernels = head["kernels"]
    dom_name = "attn_fwd"
    if headline_bwd and kernels["attn_bwd_kv"]["ms_per_step"] > kernels["attn_fwd"]["ms_per_step"]:
        dom_name = "attn_bwd_kv"
    dom = kernels[dom_name]
    line = {
        "metric": "Effective TFLOP/s (unmasked pairs only) + % of bf16 MFMA peak, 128K packed",
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_peak": head["pct_of_peak"],
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
            "useful_flop_per_step": head["useful_flop_per_step"],
            "flop_per_pair_per_head": head["flop_per_pair_per_head"],
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
            "traffic": dom.get("traffic"),
            "launches_per_step": dom["launches_per_step"],
            "avg_launch_ms": dom["avg_launch_ms"],
        },
        "kernels": kernels,
    }
    kv_steps = [s.kv_segs for s in w.steps]
    if len(rf.active) > 1 and not headline_bwd:
        # the headline step's launches one by one: each non-empty ring step's
        # useful FLOP, time and rate (step 0 writes, later steps merge)
        def by_step(tm):
            for n, i in enumerate(rf.active):
                f = sap.sap_attn_fwd if n == 0 else sap.sap_attn_fwd_merge
                tm.run(i, lambda: f(rf.plans[i], r.q, r.k, r.v, r.qs, r.ks, w.hq, w.hkv, w.d, w.scale, rf.o, rf.lse))
        tm_s, _ = _timed(a, stream, by_step)
        line["ring_steps"] = []
        for i in rf.active:
            inf = rf.infos[i]
            f_i = inf["useful_pairs_per_head"] * w.hq * FWD_PER_D * w.d
            ms_i = tm_s.ms(i) / a.steps
            line["ring_steps"].append({"step": i, "touched_q_tiles": inf["n_touched_q_tiles"], "tiles": inf["n_tiles"],
                                       "useful_flop": f_i, "ms": round(ms_i, 4),
                                       "tflops": round(f_i / (ms_i * 1e-3) / 1e12, 1)})
        # the same forward as one call over all steps' KV (a rank holding every
        # chunk), and as two calls (own chunks, then every remote chunk merged)
        for key, form, what in (("forward_single_call", "one",
                                 "forward as one call over every step's KV segments (all chunks resident; no merge)"),
                                ("forward_local_then_remote", "two",
                                 "forward as two calls: the rank's own chunks, then all remote chunks at once (merge "
                                 "in the epilogue)")):
            rr = _Rank(w, t, False, form)
            tm_c, ms_c = _timed(a, stream, lambda tm: rr.step(tm, False))
            rep = rr.report(a, tm_c, ms_c, False, what)
            line[key] = {"step": what, "value": rep["value"], "unit": "TFLOP/s", "ms_per_step": rep["ms_per_step"],
                         "kernels": {"attn_fwd": rep["kernels"]["attn_fwd"]}}
            rr.close()
        # reference: the same forward with a separate merge pass per step
        tm_2, ms_2 = _timed(a, stream, lambda tm: r.step(tm, False, fused=False))
        rep = r.report(a, tm_2, ms_2, False, "forward (ring steps + separate lse_merge pass per step)")
        line["forward_two_pass"] = {"step": rep["step"], "value": rep["value"], "unit": "TFLOP/s",
                                    "ms_per_step": rep["ms_per_step"], "kernels": rep["kernels"]}
    if with_bwd and not headline_bwd:
        if len(rf.active) > 1:
            for key, form, what in (("training_step_single_call", "one",
                                     "forward + backward as one call each over every step's KV segments (all chunks "
                                     "resident)"),
                                    ("training_step_local_then_remote", "two",
                                     "forward + backward as two calls each: the rank's own chunks, then all remote "
                                     "chunks at once")):
                rr = _Rank(w, t, True, form)
                tm_c, ms_c = _timed(a, stream, lambda tm: rr.step(tm, True))
                line[key] = rr.report(a, tm_c, ms_c, True, what)
                rr.close()
        # the same shard's training step: forward + recompute backward
        tm_t, ms_t = _timed(a, stream, lambda tm: r.step(tm, True))
        line["training_step"] = r.report(a, tm_t, ms_t, True, "forward (ring steps, fused merges) + recompute "
                                                              "backward (row terms, then per step the dK/dV pass and "
                                                              "the dQ pass)")
    if not a.no_ranks and not a.forward_only and "p" in w.extra and "chunk" in w.extra:
        line["ranks"] = rank_sweep(w, t, a, stream)
    r.close()
    del r
    torch.cuda.empty_cache()
    if not a.no_workloads:
        line["workloads"] = other_workloads(a, stream, a.workload)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, t)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Helpers shared by the GPU parity tests (not a test module).

Inputs come from the seeded ``workloads`` module; expected values only from
the fp64 ``oracle`` run on the same bf16-rounded inputs.
"""
import functools
import sys

import numpy as np
import pytest

import workloads as W

TOL_O = 2e-2      # max-abs on O, dQ, dK, dV (bf16 inputs, fp32 accumulate)
TOL_LSE = 1e-3    # max-abs on finite LSE; -inf must match exactly


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_dev(bits: np.ndarray):
    """uint16 bf16 bit patterns -> torch bfloat16 on cuda."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def f64(bits: np.ndarray) -> np.ndarray:
    return W.bf16_to_f32(bits).astype(np.float64)


@functools.lru_cache(maxsize=2)
def tensors(name: str, with_do: bool = False):
    return W.make_tensors(W.by_name(name), with_do=with_do)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, rows=None, label=""):
    """Max-abs comparison on the given local rows (all if None)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    if rows is not None:
        o_gpu, o_ref = o_gpu[rows], o_ref[rows]
        lse_gpu, lse_ref = lse_gpu[:, rows], lse_ref[:, rows]
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), ~fin), f"{label}: -inf pattern of LSE differs"
    assert not np.isnan(o_gpu).any(), f"{label}: NaN in O"
    eo = float(np.abs(o_gpu - o_ref).max()) if o_ref.size else 0.0
    el = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    say(f"  {label}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O, f"{label}: O error {eo}"
    assert el <= TOL_LSE, f"{label}: LSE error {el}"
    return eo, el


def ulysses_rows(cu, n_long: int = 2, tail: int = 256, n_random: int = 4096, seed: int = 5) -> np.ndarray:
    """The full-size sample of the 512K Ulysses shard: every row of every
    short document, and the last ``tail`` rows plus ``n_random`` seeded rows
    of each of the ``n_long`` long documents (rows are independent in the
    forward, so each sampled row is checked exactly)."""
    rng = np.random.default_rng(seed)
    rows = set()
    for i in range(len(cu) - 1):
        s, e = int(cu[i]), int(cu[i + 1])
        if i < n_long:
            rows.update(range(max(s, e - tail), e))
            rows.update(rng.integers(s, e, size=n_random).tolist())
        else:
            rows.update(range(s, e))
    return np.array(sorted(rows), dtype=np.int64)


def sample_rows(q_global: np.ndarray, cu: np.ndarray, n_random: int = 256, seed: int = 5) -> np.ndarray:
    """Local rows to check at full size: rows at and next to every document
    start inside the shard, both ends of every 128-row tile, and seeded
    random rows."""
    rng = np.random.default_rng(seed)
    tq = len(q_global)
    pos = {g: r for r, g in enumerate(q_global.tolist()) if g >= 0}
    rows = set()
    for s in cu[:-1].tolist():
        for g in (s - 1, s, s + 1):
            if g in pos:
                rows.add(pos[g])
    for t in range(0, tq, 128):
        rows.update((t, min(tq - 1, t + 127)))
    rows.update(rng.integers(0, tq, size=min(n_random, tq)).tolist())
    rows = np.array(sorted(r for r in rows if q_global[r] >= 0), dtype=np.int64)
    return rows


def oracle_workers() -> int:
    """Threads for running the oracle on independent pieces at once: the
    host's cores, at most 16 (a GPU machine's share)."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def par_map(fn, items, label=""):
    """fn over items on a thread pool with one BLAS thread per worker (NumPy
    releases the GIL inside its matrix products and ufunc loops, so the
    oracle's pieces run in parallel). Returns the results in order and says
    how far it got, so a long oracle run is visibly alive."""
    import contextlib
    import time
    from concurrent.futures import ThreadPoolExecutor, as_completed
    try:
        from threadpoolctl import threadpool_limits
        blas_one = threadpool_limits(limits=1, user_api="blas")
    except Exception:
        blas_one = contextlib.nullcontext()
    t0 = last = time.perf_counter()
    out = [None] * len(items)
    with blas_one, ThreadPoolExecutor(max_workers=oracle_workers()) as ex:
        futs = {ex.submit(fn, it): i for i, it in enumerate(items)}
        done = 0
        for f in as_completed(futs):
            out[futs[f]] = f.result()
            done += 1
            now = time.perf_counter()
            if label and (done == len(items) or now - last >= 10.0):
                last = now
                say(f"  oracle {label}: {done}/{len(items)} pieces, {now - t0:.1f} s")
    return out


def oracle_forward_rows(q, k, v, gq, gk, cu, scale, rows, label="", piece=256):
    """The oracle forward on the given local Q rows only (each row is
    independent, so computing them in pieces is exact): returns O [len(rows),
    Hq, D] and LSE [Hq, len(rows)] in the order of ``rows``. q, k, v may be
    bf16 bit patterns (uint16) or floats."""
    from oracle import attention as A
    rows = np.asarray(rows, dtype=np.int64)
    conv = lambda x: f64(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float64)
    k64, v64 = conv(k), conv(v)
    gq = np.asarray(gq, dtype=np.int64)
    pieces = [rows[i:i + piece] for i in range(0, len(rows), piece)]

    def one(rs):
        return A.forward(conv(q[rs]), k64, v64, gq[rs], gk, cu, scale)

    res = par_map(one, pieces, label)
    if not res:
        hq, d = q.shape[1], q.shape[2]
        return np.zeros((0, hq, d)), np.zeros((hq, 0))
    return np.concatenate([r[0] for r in res], axis=0), np.concatenate([r[1] for r in res], axis=1)


def oracle_fwd_bwd_full(q, k, v, do, gq, cu, scale, label="", max_rows=1024):
    """The oracle's forward and backward of a rank at full size, every row:
    q, do local rows [Tq, Hq, D], k, v whole-sequence [T, Hkv, D] (bf16 bit
    patterns or floats), gq the global position of every local row. The
    forward runs in pieces of rows; the backward in (KV head, document, block
    of <= max_rows query rows) pieces, which is exact: a dQ row is a sum over
    its own document's keys, and a key's dK / dV is the sum of the pieces'
    partial sums over that document's rows (added here in a fixed order).
    Returns O, LSE, dQ, dK, dV in float64."""
    from oracle import attention as A
    conv = lambda x: f64(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float64)
    gq = np.asarray(gq, dtype=np.int64)
    cu = np.asarray(cu, dtype=np.int64)
    tq, hq = q.shape[0], q.shape[1]
    total, hkv, d = k.shape
    grp = hq // hkv
    k64, v64 = conv(k), conv(v)
    o, lse = oracle_forward_rows(q, k64, v64, gq, np.arange(total), cu, scale, np.arange(tq), label=f"{label} fwd")
    doc_q = np.searchsorted(cu, gq, side="right") - 1
    pieces = []
    for g in range(hkv):
        for dd in np.unique(doc_q):
            rows = np.nonzero(doc_q == dd)[0]
            for i in range(0, len(rows), max_rows):
                pieces.append((g, int(dd), rows[i:i + max_rows]))

    def one(piece):
        g, dd, rows = piece
        hs = slice(g * grp, (g + 1) * grp)
        keys = np.arange(cu[dd], cu[dd + 1])
        return A.backward(conv(q[rows][:, hs]), k64[keys, g:g + 1], v64[keys, g:g + 1], conv(do[rows][:, hs]),
                          o[rows][:, hs], lse[hs][:, rows], gq[rows], keys, cu, scale)

    res = par_map(one, pieces, label=f"{label} bwd")
    dq = np.zeros((tq, hq, d))
    dk = np.zeros((total, hkv, d))
    dv = np.zeros((total, hkv, d))
    for (g, dd, rows), (pq, pk, pv) in zip(pieces, res):
        hs = slice(g * grp, (g + 1) * grp)
        keys = slice(int(cu[dd]), int(cu[dd + 1]))
        dq[rows, hs] = pq
        dk[keys, g:g + 1] += pk
        dv[keys, g:g + 1] += pv
    return o, lse, dq, dk, dv


def balanced_rank3():
    """Rank 3 of the 128K sequence in the document-aware balanced layout
    (1024-row chunks), the chunk owners taken from the oracle's assignment."""
    from oracle import balance as B
    z = W.zigzag_rank(3)
    owner = B.balance(z.cu, 8, 1024)[0]
    return W.owner_rank(z, list(owner), 3, 1024, "balanced")


@functools.lru_cache(maxsize=3)
def full_reference(name: str):
    """The oracle's O, LSE, dQ, dK, dV of a named workload's rank on every row
    and key (computed once per test process and shared by the tests of its
    different schedules, which must all reproduce it). ``balanced`` is rank 3
    of the 128K sequence in the balanced layout (inputs of ``zigzag``)."""
    w = balanced_rank3() if name == "balanced" else W.by_name(name)
    t = tensors("zigzag" if name == "balanced" else name, True)
    say(f"  oracle reference of {w.name}: every row and key, forward and backward")
    ql, dol = W.local_rows(t.q, w.q_segs), W.local_rows(t.do, w.q_segs)
    return oracle_fwd_bwd_full(ql, t.k, t.v, dol, w.q_global_rows(), w.cu, w.scale, label=w.name)

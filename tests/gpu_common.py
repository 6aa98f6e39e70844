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

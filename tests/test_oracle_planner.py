"""Pins for the oracle planner (non-empty tiles and their FULL/DIAGONAL/PARTIAL class).

The closed interval rules are checked against the brute-force reading of
each tile's dense mask (all-false -> omitted, all-true -> FULL, equal to the
plain causal mask -> DIAGONAL, else PARTIAL), and the useful-pair count
against the closed form sum over documents of L(L+1)/2.
"""
import numpy as np
import pytest

import workloads as W
from oracle import planner as P


def _positions(tiles):
    return [np.arange(g, g + n) for _, n, g in tiles]


def _dense_doc_mask(cu, gq, gk):
    """Mask from explicit document ids (independent of the oracle's ds() helper)."""
    cu = np.asarray(cu)
    total = int(cu[-1])
    doc_id = np.empty(total, dtype=np.int64)
    for i in range(len(cu) - 1):
        doc_id[cu[i]:cu[i + 1]] = i
    return (doc_id[gq][:, None] == doc_id[gk][None, :]) & (gk[None, :] <= gq[:, None])


def brute_plan(cu, q_segs, kv_segs, bm, bn):
    qt = P.tiles_of(q_segs, bm)
    kt = P.tiles_of(kv_segs, bn)
    qpos, kpos = _positions(qt), _positions(kt)
    out = []
    useful = 0
    for i, gq in enumerate(qpos):
        for j, gk in enumerate(kpos):
            m = _dense_doc_mask(cu, gq, gk)
            if not m.any():
                continue
            causal = gk[None, :] <= gq[:, None]
            cls = P.FULL if m.all() else (P.DIAGONAL if np.array_equal(m, causal) else P.PARTIAL)
            out.append((i, j, cls))
            useful += int(m.sum())
    return out, useful


def _as_list(pl):
    return list(zip(pl.q_tile.tolist(), pl.kv_tile.tolist(), pl.cls.tolist()))


def test_tiny_against_brute_force():
    w = W.tiny()
    pl = P.plan(w.cu, w.q_segs, w.steps[0].kv_segs, 128, 64)
    ref, useful = brute_plan(w.cu, w.q_segs, w.steps[0].kv_segs, 128, 64)
    assert _as_list(pl) == ref
    assert pl.useful_pairs == useful == sum(L * (L + 1) // 2 for L in w.lengths)


@pytest.mark.parametrize("seed", range(12))
def test_random_layouts_against_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    p = int(rng.choice([1, 2, 4]))
    chunk = int(rng.integers(8, 200))
    zig = bool(rng.integers(0, 2)) and p > 1
    nch = 2 * p if zig else p
    total = nch * chunk
    lengths = W.random_docs(rng, total, int(rng.integers(2, 3 * chunk)))
    cu = W.cu_seqlens(lengths)
    bm = int(rng.choice([16, 32, 64, 128]))
    bn = int(rng.choice([16, 32, 64, 128]))
    rank = int(rng.integers(0, p))
    if zig:
        jj = 2 * p - 1 - rank
        q_segs = [(rank * chunk, (rank + 1) * chunk, 0), (jj * chunk, (jj + 1) * chunk, chunk)]
    else:
        q_segs = [(rank * chunk, (rank + 1) * chunk, 0)]
    per_row = 0
    for s in range(p):
        j = (rank - s) % p
        if zig:
            j2 = 2 * p - 1 - j
            kv = [(j * chunk, (j + 1) * chunk, j * chunk), (j2 * chunk, (j2 + 1) * chunk, j2 * chunk)]
        else:
            kv = [(j * chunk, (j + 1) * chunk, 0)]
        pl = P.plan(cu, q_segs, kv, bm, bn)
        ref, useful = brute_plan(cu, q_segs, kv, bm, bn)
        assert _as_list(pl) == ref
        assert pl.useful_pairs == useful
        per_row += useful
    # over all steps every local query sees exactly its causal document prefix
    gq = np.concatenate([np.arange(gs, ge) for gs, ge, _ in q_segs])
    ds = cu[np.searchsorted(cu, gq, side="right") - 1]
    assert per_row == int((gq - ds + 1).sum())


def test_non_empty_kv_tiles_are_one_interval_per_q_tile():
    rng = np.random.default_rng(7)
    lengths = W.random_docs(rng, 3000, 400)
    cu = W.cu_seqlens(lengths)
    pl = P.plan(cu, [(0, 3000, 0)], [(0, 3000, 0)], 64, 32)
    for qt in np.unique(pl.q_tile):
        sel = pl.q_tile == qt
        kv = pl.kv_tile[sel]
        assert (np.diff(kv) == 1).all()
        full = kv[pl.cls[sel] == P.FULL]
        if len(full):
            assert (np.diff(full) == 1).all()


def test_ragged_and_empty_segments():
    cu = W.cu_seqlens([5, 0, 70, 1, 24])
    q_segs = [(0, 37, 3), (37, 37, 40), (60, 100, 50)]      # an empty segment, gaps in local rows
    kv_segs = [(0, 100, 0)]
    pl = P.plan(cu, q_segs, kv_segs, 16, 16)
    ref, useful = brute_plan(cu, q_segs, kv_segs, 16, 16)
    assert _as_list(pl) == ref and pl.useful_pairs == useful
    assert [t[0] for t in pl.q_tiles] == [3, 19, 35, 50, 66, 82]
    assert [t[1] for t in pl.q_tiles] == [16, 16, 5, 16, 16, 8]


def test_golden_tiny_tile_list():
    """Regression pin: the stored list was written by tests/golden/make_golden.py (oracle only)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_tiles_128x64.txt")
    rows = [tuple(int(x) for x in line.split()) for line in open(path)
            if line.strip() and not line.startswith("#")]
    w = W.tiny()
    pl = P.plan(w.cu, w.q_segs, w.steps[0].kv_segs, 128, 64)
    assert _as_list(pl) == rows

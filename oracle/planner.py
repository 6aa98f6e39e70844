"""fp64/int reference planner: non-empty (Q-tile, KV-tile) pairs and their mask class.

Test infrastructure only. This is the one-device form of the schedule the HSAP
summary page (gptget.net/papers/2606.30460, method section and technical
contributions) generates ahead of time for irregular attention: only blocks
that hold at least one allowed (query, key) pair are listed.

Tiling. A segment (gs, ge, ls) maps global positions [gs, ge) to local rows
ls, ls+1, ... Query tiles are runs of BM local rows starting at each Q
segment's local start; the last run of a segment may be shorter. They are
numbered consecutively over the segments in local-row order. KV tiles are
runs of BN rows built and numbered the same way over the KV segments. A tile
therefore never straddles a segment, so its rows are consecutive global
positions.

Classes, for a Q tile with global positions [a, b] and a KV tile [c, e]
(ds(p) = start of the document holding p):

    EMPTY    <=> c > b  or  e < ds(a)         (not listed)
    FULL     <=> e <= a  and  c >= ds(b)      (every pair allowed)
    DIAGONAL <=> not FULL and c >= ds(b)      (mask is exactly key <= query)
    PARTIAL  otherwise                        (a document start lies inside)

These closed rules are pinned in the tests against the brute-force reading
on the dense tile mask: all-false -> EMPTY, all-true -> FULL, equal to the
plain causal mask -> DIAGONAL, else PARTIAL.

Listing order: q_tile ascending, then kv_tile ascending; the list is unique.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .attention import doc_start

FULL, DIAGONAL, PARTIAL = 0, 1, 2


def tiles_of(segs, b):
    """[(local_start, n_rows, global_start)] of the b-row tiles of a segment table."""
    out = []
    for gs, ge, ls in sorted(segs, key=lambda s: s[2]):
        for off in range(0, ge - gs, b):
            out.append((ls + off, min(b, ge - gs - off), gs + off))
    return out


@dataclass
class Plan:
    q_tiles: list        # (local_start, n, global_start) per Q tile
    kv_tiles: list       # (local_start, n, global_start) per KV tile
    q_tile: np.ndarray   # int32 [n]
    kv_tile: np.ndarray  # int32 [n]
    cls: np.ndarray      # uint8 [n]
    useful_pairs: int    # allowed (query, key) pairs per head over the listed tiles

    @property
    def touched(self) -> np.ndarray:
        return np.unique(self.q_tile).astype(np.int32)

    @property
    def n_tiles(self) -> int:
        return len(self.q_tile)


def plan(cu, q_segs, kv_segs, bm, bn) -> Plan:
    cu = np.asarray(cu, dtype=np.int64)
    qt = tiles_of(q_segs, bm)
    kt = tiles_of(kv_segs, bn)
    if not kt:
        e32 = np.zeros(0, dtype=np.int32)
        return Plan(qt, kt, e32, e32.copy(), np.zeros(0, dtype=np.uint8), 0)
    k_lo = np.array([g for _, _, g in kt], dtype=np.int64)
    k_hi = k_lo + np.array([n for _, n, _ in kt], dtype=np.int64) - 1
    kidx = np.arange(len(kt), dtype=np.int32)
    q_out, k_out, c_out = [], [], []
    useful = 0
    for ti, (_, n, g0) in enumerate(qt):
        a, b = g0, g0 + n - 1
        ds_a = int(doc_start(cu, [a])[0])
        ds_b = int(doc_start(cu, [b])[0])
        nonempty = ~((k_lo > b) | (k_hi < ds_a))
        if not nonempty.any():
            continue
        full = (k_hi <= a) & (k_lo >= ds_b)
        diag = ~full & (k_lo >= ds_b)
        cls = np.where(full, FULL, np.where(diag, DIAGONAL, PARTIAL)).astype(np.uint8)
        sel = kidx[nonempty]
        q_out.append(np.full(len(sel), ti, dtype=np.int32))
        k_out.append(sel)
        c_out.append(cls[nonempty])
        # allowed pairs: every pair of a FULL tile; otherwise row p sees keys
        # [max(ds(p), lo), min(p, hi)] of the tile
        fsel = sel[full[nonempty]]
        useful += int(n * (k_hi[fsel] - k_lo[fsel] + 1).sum())
        osel = sel[~full[nonempty]]
        if len(osel):
            rows = np.arange(a, b + 1, dtype=np.int64)
            ds_rows = doc_start(cu, rows)
            lo = np.maximum(ds_rows[:, None], k_lo[osel][None, :])
            hi = np.minimum(rows[:, None], k_hi[osel][None, :])
            useful += int(np.clip(hi - lo + 1, 0, None).sum())
    if q_out:
        q_arr = np.concatenate(q_out)
        k_arr = np.concatenate(k_out)
        c_arr = np.concatenate(c_out)
    else:
        q_arr = np.zeros(0, dtype=np.int32)
        k_arr = np.zeros(0, dtype=np.int32)
        c_arr = np.zeros(0, dtype=np.uint8)
    return Plan(qt, kt, q_arr, k_arr, c_arr, useful)

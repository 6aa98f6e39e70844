"""Pins for the oracle's exact merge of partial attention results.

Sequence parallelism is computation-equivalent to one-device attention (SP
blog page, bmjup.com/post/14448.html, FAQ Q1), and a ring of KV chunks gives
every rank the full-sequence result (same page, core principles). So: any
split of the KV rows into chunks, computed separately and merged in any
order, must equal the unchunked result.
"""
import numpy as np

import workloads as W
from oracle import attention as A


def _case(rng, lengths, h=2, hkv=None, d=8):
    t = sum(lengths)
    hkv = hkv or h
    q = rng.standard_normal((t, h, d))
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    return q, k, v, W.cu_seqlens(lengths)


def _merge_all(parts, order):
    o, lse = parts[order[0]]
    for i in order[1:]:
        o, lse = A.merge(o, lse, *parts[i])
    return o, lse


def test_random_chunkings_in_any_order_equal_unchunked(rng):
    for trial in range(25):
        lengths = W.random_docs(rng, int(rng.integers(20, 160)), 40)
        q, k, v, cu = _case(rng, lengths, h=4, hkv=2)
        t = q.shape[0]
        g = np.arange(t)
        full_o, full_l = A.forward(q, k, v, g, g, cu, 0.3)
        nchunks = int(rng.integers(1, 7))
        cuts = np.sort(rng.integers(0, t + 1, size=nchunks - 1))
        bounds = np.concatenate([[0], cuts, [t]])     # may include empty chunks
        parts = []
        for a, b in zip(bounds[:-1], bounds[1:]):
            gk = np.arange(a, b)
            parts.append(A.forward(q, k[a:b], v[a:b], g, gk, cu, 0.3))
        order = rng.permutation(len(parts))
        o, lse = _merge_all(parts, order)
        assert np.abs(o - full_o).max() < 1e-12
        fin = np.isfinite(full_l)
        assert (np.isfinite(lse) == fin).all()
        assert np.abs(lse[fin] - full_l[fin]).max() < 1e-12


def test_neg_inf_partial_is_identity(rng):
    t, h, d = 12, 3, 5
    o = rng.standard_normal((t, h, d))
    lse = rng.standard_normal((h, t))
    lse[1, 4] = -np.inf
    o[4, 1] = 0.0
    o2, lse2 = A.merge(o, lse, np.zeros_like(o), np.full_like(lse, -np.inf))
    assert np.array_equal(o2, o) and np.array_equal(lse2, lse)
    o3, lse3 = A.merge(np.zeros_like(o), np.full_like(lse, -np.inf), o, lse)
    assert np.array_equal(o3, o) and np.array_equal(lse3, lse)


def test_two_equal_halves(rng):
    """Closed form: equal LSE on both sides gives the mean and LSE + ln 2."""
    t, h, d = 6, 2, 4
    oa, ob = rng.standard_normal((t, h, d)), rng.standard_normal((t, h, d))
    lse = rng.standard_normal((h, t))
    o, l2 = A.merge(oa, lse, ob, lse)
    assert np.abs(o - 0.5 * (oa + ob)).max() < 1e-15
    assert np.abs(l2 - (lse + np.log(2.0))).max() < 1e-14


def test_ring_steps_of_sharded_rank_equal_full(rng):
    """A rank's zigzag Q shard merged over ring steps equals attention over all KV."""
    p, chunk = 4, 16
    t = 2 * p * chunk
    lengths = W.random_docs(rng, t, 50)
    q, k, v, cu = _case(rng, lengths, h=2, d=8)
    rank = 1
    jj = 2 * p - 1 - rank
    gq = np.concatenate([np.arange(rank * chunk, (rank + 1) * chunk), np.arange(jj * chunk, (jj + 1) * chunk)])
    g = np.arange(t)
    ref_o, ref_l = A.forward(q[gq], k, v, gq, g, cu, 0.5)
    acc = None
    for s in range(p):
        j = (rank - s) % p
        gk = np.concatenate([np.arange(j * chunk, (j + 1) * chunk),
                             np.arange((2 * p - 1 - j) * chunk, (2 * p - j) * chunk)])
        part = A.forward(q[gq], k[gk], v[gk], gq, gk, cu, 0.5)
        acc = part if acc is None else A.merge(*acc, *part)
    assert np.abs(acc[0] - ref_o).max() < 1e-12
    assert np.abs(acc[1] - ref_l).max() < 1e-12

"""Pins for the oracle's document-aware chunk-to-rank assignment.

* hand-worked assignments (tests/golden/balance_hand_examples.txt), derived on
  paper from the rule, catch a wrong sort direction, tie order or room check;
* chunk work against a brute-force count of the dense document mask (built
  from explicit document ids, not the oracle's ds() helper) and against the
  closed form for one document, 4c+3 style sums k*(c*k) + k(k+1)/2;
* totals against the closed form sum over documents of L(L+1)/2;
* equal chunk works reduce the rule to round robin (chunk c -> rank c mod P);
* invariants on seeded layouts: each rank holds n_chunks / n_ranks chunks and
  its work is the sum of its chunks' works.
"""
import os

import numpy as np
import pytest

import workloads as W
from oracle import balance as B

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "balance_hand_examples.txt")


def _hand_examples():
    out = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, cu, p, k, work, owner, load = [f.strip() for f in line.split("|")]
        ints = lambda s: [int(x) for x in s.split()]
        out.append((name, ints(cu), int(p), int(k), ints(work), ints(owner), ints(load)))
    return out


@pytest.mark.parametrize("case", _hand_examples(), ids=lambda c: c[0])
def test_hand_examples(case):
    _, cu, p, k, work, owner, load = case
    assert list(B.chunk_work(cu, k)) == work
    got_owner, got_load = B.balance(cu, p, k)
    assert got_owner == owner
    assert got_load == load


def _brute_chunk_work(cu, chunk):
    cu = np.asarray(cu)
    total = int(cu[-1])
    doc_id = np.empty(total, dtype=np.int64)
    for i in range(len(cu) - 1):
        doc_id[cu[i]:cu[i + 1]] = i
    pos = np.arange(total)
    mask = (doc_id[:, None] == doc_id[None, :]) & (pos[None, :] <= pos[:, None])
    return mask.sum(axis=1).reshape(-1, chunk).sum(axis=1)


@pytest.mark.parametrize("seed", range(8))
def test_chunk_work_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    chunk = int(rng.choice([1, 4, 16, 32]))
    total = chunk * int(rng.integers(1, 24))
    lengths = W.random_docs(rng, total, max_len=total)
    cu = W.cu_seqlens(lengths)
    assert np.array_equal(B.chunk_work(cu, chunk), _brute_chunk_work(cu, chunk))


def test_chunk_work_one_document_closed_form():
    k, n = 8, 32
    work = B.chunk_work([0, k * n], k)
    expect = [k * (c * k) + k * (k + 1) // 2 for c in range(n)]
    assert list(work) == expect


@pytest.mark.parametrize("name", ["ring", "zigzag", "train"])
def test_total_work_closed_form(name):
    w = W.by_name(name)
    work = B.chunk_work(w.cu, 1024)
    assert int(work.sum()) == sum(L * (L + 1) // 2 for L in w.lengths)


def test_equal_work_is_round_robin():
    k, p, n = 16, 4, 32
    cu = [k * i for i in range(n + 1)]  # every chunk is one whole document
    owner, load = B.balance(cu, p, k)
    assert owner == [c % p for c in range(n)]
    assert load == [(n // p) * k * (k + 1) // 2] * p


@pytest.mark.parametrize("seed", range(6))
def test_invariants(seed):
    rng = np.random.default_rng(200 + seed)
    p = int(rng.choice([2, 3, 4, 8]))
    chunk = int(rng.choice([4, 16, 64]))
    total = p * chunk * int(rng.integers(1, 9))
    cu = W.cu_seqlens(W.random_docs(rng, total, max_len=total))
    owner, load = B.balance(cu, p, chunk)
    work = B.chunk_work(cu, chunk)
    n = total // chunk
    assert sorted(owner) == sorted([r for r in range(p) for _ in range(n // p)])
    for r in range(p):
        assert load[r] == int(work[[c for c in range(n) if owner[c] == r]].sum())


def test_balanced_beats_zigzag_on_the_128k_sequence():
    """The 128K zigzag layout leaves a large spread of work; the balanced one nearly none."""
    w = W.zigzag_rank(3)
    p = w.extra["p"]
    zz = B.chunk_work(w.cu, w.extra["chunk"])
    zz_load = [int(zz[r] + zz[2 * p - 1 - r]) for r in range(p)]
    _, load = B.balance(w.cu, p, 1024)
    assert sum(load) == sum(zz_load)
    assert max(zz_load) / min(zz_load) > 3.0
    assert max(load) / (sum(load) / p) < 1.01


def test_rejects_bad_sizes():
    with pytest.raises(ValueError):
        B.balance([0, 10], 2, 4)

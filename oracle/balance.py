"""Reference document-aware assignment of query chunks to sequence-parallel ranks.

Test infrastructure only (see the package docstring).

Why. With packed documents a token's attention work is the length of its
window [ds(i), i], so equal token counts per rank do not give equal work:
the SP blog page (bmjup.com/post/14448.html, section on future trends and
challenges) names uneven sequence lengths leaving some GPUs idle, and the
HSAP summary page (gptget.net/papers/2606.30460, technical contributions)
balances load across devices by scheduling. The pages give no algorithm.
The reading taken here is the plainest one that keeps every rank's token
count (and so its activation memory) equal:

* the sequence is cut into chunks of ``chunk`` consecutive positions;
* a chunk's work is the number of allowed (query, key) pairs of its rows,
  sum over its positions i of (i - ds(i) + 1);
* chunks are assigned greedily, heaviest first (ties: lower chunk index
  first), each to the rank with the least work so far among the ranks that
  hold fewer than n_chunks / n_ranks chunks (ties: lower rank first).
  This is the longest-processing-time rule with a cardinality limit.

Each rank then holds its chunks in ascending position order.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

from .attention import doc_start


def chunk_work(cu, chunk: int) -> np.ndarray:
    """Allowed (query, key) pairs per head of every chunk, row by row."""
    cu = np.asarray(cu, dtype=np.int64)
    total = int(cu[-1])
    pos = np.arange(total, dtype=np.int64)
    per_row = pos - doc_start(cu, pos) + 1
    return per_row.reshape(total // chunk, chunk).sum(axis=1)


def balance(cu, n_ranks: int, chunk: int) -> Tuple[List[int], List[int]]:
    """Owner rank of every chunk and the resulting work per rank."""
    total = int(np.asarray(cu)[-1])
    if chunk < 1 or n_ranks < 1 or total % (chunk * n_ranks) != 0:
        raise ValueError("total length must be a multiple of chunk * n_ranks")
    work = [int(x) for x in chunk_work(cu, chunk)]
    n_chunks = len(work)
    cap = n_chunks // n_ranks
    order = sorted(range(n_chunks), key=lambda c: (-work[c], c))
    load = [0] * n_ranks
    count = [0] * n_ranks
    owner = [-1] * n_chunks
    for c in order:
        best = -1
        for r in range(n_ranks):
            if count[r] < cap and (best < 0 or load[r] < load[best]):
                best = r
        owner[c] = best
        load[best] += work[c]
        count[best] += 1
    return owner, load

"""Seeded synthetic workloads for document-masked (packed) causal attention.

This module is shared by the oracle's tests, the GPU parity tests and the
benchmark. It only *describes* inputs: document lengths, the rows a
sequence-parallel rank holds, the KV chunks each ring step brings, and seeded
tensors rounded to bfloat16. It holds none of the attention arithmetic.

Workloads stand in for the "hybrid-context packed sequences" of 128K-512K
tokens that the HSAP summary page (gptget.net/papers/2606.30460, key results
and original abstract) trains on. The pages name no dataset, so document
lengths are drawn from seeded distributions and tensors are N(0, 1):

* log-uniform lengths on [a, b]:  L = min(max(floor(exp(U(ln a, ln(b+1)))), a), b)
  with ``numpy.random.default_rng(seed)``; draws continue until the running
  sum reaches T, and the last length is cut so the sum is exactly T.
* the Ulysses shard: two long documents (262144, 131072) first, then
  ``rng.integers(64, 2049)`` draws with the same cut.
* tensors: ``default_rng(seed).standard_normal((T, H, D), float32)`` over the
  whole sequence, rounded to bf16 with round-to-nearest-even; seeds Q=1, K=2,
  V=3, dO=4. A rank's Q (and dO) are row slices; K/V stay whole-sequence and
  each ring step views its chunks in place.

Sequence-parallel layouts follow the SP blog page (bmjup.com/post/14448.html,
section on core principles: each GPU holds one contiguous token chunk and the
KV chunks travel round a ring). The ring direction is not given there: here
rank r at step s holds the chunk that started on rank (r - s) mod P. The
zigzag layout (rank r owns chunks r and 2P-1-r) is not on the pages; it is
the load-balanced chunking used for the 128K GQA shard.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

SEED_LENGTHS = 0
SEED_Q, SEED_K, SEED_V, SEED_DO = 1, 2, 3, 4

# A segment maps global positions [global_start, global_end) of the packed
# sequence onto local rows local_start, local_start+1, ... of a buffer.
Segment = Tuple[int, int, int]


def loguniform_lengths(total: int, lo: int, hi: int, seed: int = SEED_LENGTHS) -> List[int]:
    rng = np.random.default_rng(seed)
    out: List[int] = []
    s = 0
    while s < total:
        u = rng.uniform(math.log(lo), math.log(hi + 1))
        length = min(max(int(math.floor(math.exp(u))), lo), hi)
        if s + length >= total:
            length = total - s
        out.append(length)
        s += length
    return out


def ulysses_lengths(total: int = 524288, seed: int = SEED_LENGTHS) -> List[int]:
    out = [262144, 131072]
    s = sum(out)
    rng = np.random.default_rng(seed)
    while s < total:
        length = int(rng.integers(64, 2049))
        if s + length >= total:
            length = total - s
        out.append(length)
        s += length
    return out


def cu_seqlens(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs are finite normals, so NaN handling is not needed."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def seeded_bf16(shape, seed: int) -> np.ndarray:
    """N(0,1) fp32 from ``default_rng(seed)`` rounded to bf16; returns uint16 bits."""
    rng = np.random.default_rng(seed)
    return bf16_round(rng.standard_normal(shape, dtype=np.float32))


@dataclass
class Step:
    """One call's KV set: the chunks a rank holds at one ring step."""
    index: int
    chunks: List[int]
    kv_segs: List[Segment]


@dataclass
class Workload:
    name: str
    description: str
    lengths: List[int]
    hq: int
    hkv: int
    d: int
    q_segs: List[Segment]
    steps: List[Step]
    backward: bool = False
    input_dtype: str = "bf16"
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def total(self) -> int:
        return int(sum(self.lengths))

    @property
    def cu(self) -> np.ndarray:
        return cu_seqlens(self.lengths)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def tq(self) -> int:
        return max(ls + (ge - gs) for gs, ge, ls in self.q_segs)

    def q_global_rows(self) -> np.ndarray:
        """Global position of every local Q row (segments in local order)."""
        g = np.full(self.tq, -1, dtype=np.int64)
        for gs, ge, ls in self.q_segs:
            g[ls:ls + (ge - gs)] = np.arange(gs, ge)
        return g


def _ring_steps(p: int, rank: int, chunk: int) -> List[Step]:
    steps = []
    for s in range(p):
        j = (rank - s) % p
        steps.append(Step(s, [j], [(j * chunk, (j + 1) * chunk, j * chunk)]))
    return steps


def _zigzag_steps(p: int, rank: int, chunk: int) -> List[Step]:
    steps = []
    for s in range(p):
        j = (rank - s) % p
        jj = 2 * p - 1 - j
        segs = sorted([(j * chunk, (j + 1) * chunk, j * chunk),
                       (jj * chunk, (jj + 1) * chunk, jj * chunk)], key=lambda t: t[2])
        steps.append(Step(s, [j, jj], segs))
    return steps


def _runs(chunks: List[int], chunk: int, local: bool) -> List[Segment]:
    """Segments of ascending chunk indices, consecutive chunks merged.

    local=True packs them into consecutive local rows from 0 (a rank's own
    buffer); local=False keeps local row = global position (a whole-sequence
    buffer viewed in place)."""
    segs: List[Segment] = []
    ls = 0
    for c in sorted(chunks):
        gs, ge = c * chunk, (c + 1) * chunk
        if segs and segs[-1][1] == gs:
            segs[-1] = (segs[-1][0], ge, segs[-1][2])
        else:
            segs.append((gs, ge, ls if local else gs))
        ls += chunk
    return segs


def zigzag_owner(p: int) -> List[int]:
    """Owner rank of each of the 2P chunks of the zigzag layout (r owns r and 2P-1-r)."""
    return [j if j < p else 2 * p - 1 - j for j in range(2 * p)]


def owner_rank(base: "Workload", owner: List[int], rank: int, chunk: int, tag: str) -> "Workload":
    """The workload of one rank of a chunk-to-rank layout given as ``owner[c]``.

    The rank holds its chunks' Q rows in ascending order; at ring step s it
    holds the KV chunks of rank (rank - s) mod P, viewed in place in the
    whole-sequence K/V (the same ring direction as the other layouts)."""
    p = max(owner) + 1
    mine = [c for c, r in enumerate(owner) if r == rank]
    steps = []
    for s in range(p):
        src = (rank - s) % p
        theirs = [c for c, r in enumerate(owner) if r == src]
        steps.append(Step(s, theirs, _runs(theirs, chunk, local=False)))
    return Workload(f"{tag}_rank{rank}", f"{base.description}, {tag} layout",
                    base.lengths, base.hq, base.hkv, base.d, _runs(mine, chunk, local=True), steps,
                    extra={"p": p, "rank": rank, "chunk": chunk, "layout": tag})


def tiny() -> Workload:
    lengths = [64, 192, 32, 224]
    return Workload("tiny_packed_512", "512 tokens, 4 documents, 2 heads, head_dim 64, P=1",
                    lengths, 2, 2, 64, [(0, 512, 0)], [Step(0, [0], [(0, 512, 0)])],
                    input_dtype="fp32",
                    notes="fp32 N(0,1) inputs; the bf16 path sees them rounded to bf16")


def ring_rank(rank: int = 3) -> Workload:
    total, p = 32768, 8
    chunk = total // p
    lengths = loguniform_lengths(total, 128, 8192)
    return Workload(f"ring_sp8_32k_rank{rank}", "32768 tokens, SP=8 ring, 32 heads, head_dim 128",
                    lengths, 32, 32, 128, [(rank * chunk, (rank + 1) * chunk, 0)],
                    _ring_steps(p, rank, chunk), extra={"p": p, "rank": rank, "chunk": chunk})


def zigzag_rank(rank: int = 3) -> Workload:
    total, p = 131072, 8
    chunk = total // (2 * p)
    lengths = loguniform_lengths(total, 256, 32768)
    jj = 2 * p - 1 - rank
    q_segs = [(rank * chunk, (rank + 1) * chunk, 0), (jj * chunk, (jj + 1) * chunk, chunk)]
    return Workload(f"zigzag_sp8_128k_gqa_rank{rank}",
                    "131072 tokens, SP=8 zigzag, 32 query / 8 KV heads, head_dim 128",
                    lengths, 32, 8, 128, q_segs, _zigzag_steps(p, rank, chunk),
                    extra={"p": p, "rank": rank, "chunk": chunk})


def ulysses(hkv: int = 4) -> Workload:
    """One Ulysses rank: the whole 512K sequence for its 4 query heads.

    hkv=4 is the plain head split; hkv=1 is a GQA-aware split of a 32-query /
    8-KV-head model over 8 ranks, where each rank keeps one KV group (4 query
    heads sharing one KV head) and so needs one KV head only."""
    lengths = ulysses_lengths()
    total = sum(lengths)
    name = "ulysses_512k_4heads" if hkv == 4 else f"ulysses_512k_4q{hkv}kv"
    desc = "524288 tokens, hybrid context, 4 heads, head_dim 128" if hkv == 4 else \
        f"524288 tokens, hybrid context, 4 query heads / {hkv} KV head(s), head_dim 128"
    return Workload(name, desc, lengths, 4, hkv, 128, [(0, total, 0)], [Step(0, [0], [(0, total, 0)])])


def training() -> Workload:
    lengths = loguniform_lengths(65536, 1, 16384)
    return Workload("train_64k_5heads", "65536 tokens, 5 heads, head_dim 128, fwd+bwd",
                    lengths, 5, 5, 128, [(0, 65536, 0)], [Step(0, [0], [(0, 65536, 0)])],
                    backward=True)


ALL = {"tiny": tiny, "ring": ring_rank, "zigzag": zigzag_rank, "ulysses": ulysses,
       "ulysses_gqa": lambda: ulysses(hkv=1), "train": training}


def by_name(name: str, **kw) -> Workload:
    return ALL[name](**kw)


@dataclass
class Tensors:
    """Whole-sequence inputs as bf16 bit patterns (uint16) plus their fp32 widening."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray] = None


def make_tensors(w: Workload, with_do: bool = False) -> Tensors:
    """Seeded inputs over the whole packed sequence (Q/dO: Hq heads, K/V: Hkv)."""
    t = w.total
    if w.input_dtype == "fp32":
        # fp32 N(0,1); the bf16 kernels consume the RNE-rounded values.
        def gen(h, seed):
            return bf16_round(np.random.default_rng(seed).standard_normal((t, h, w.d), dtype=np.float32))
    else:
        def gen(h, seed):
            return seeded_bf16((t, h, w.d), seed)
    q = gen(w.hq, SEED_Q)
    k = gen(w.hkv, SEED_K)
    v = gen(w.hkv, SEED_V)
    do = gen(w.hq, SEED_DO) if with_do else None
    return Tensors(q, k, v, do)


def fp32_inputs_tiny() -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The tiny workload's unrounded fp32 inputs (for reporting the bf16 input error)."""
    w = tiny()
    gen = lambda h, s: np.random.default_rng(s).standard_normal((w.total, h, w.d), dtype=np.float32)
    return gen(w.hq, SEED_Q), gen(w.hkv, SEED_K), gen(w.hkv, SEED_V)


def local_rows(bits: np.ndarray, segs: List[Segment], nrows: Optional[int] = None) -> np.ndarray:
    """Gather a rank's local buffer from whole-sequence rows by its segment table."""
    n = nrows if nrows is not None else max(ls + (ge - gs) for gs, ge, ls in segs)
    out = np.zeros((n,) + bits.shape[1:], dtype=bits.dtype)
    for gs, ge, ls in segs:
        out[ls:ls + (ge - gs)] = bits[gs:ge]
    return out


def random_docs(rng: np.random.Generator, total: int, max_len: int, p_one: float = 0.15,
                p_empty: float = 0.05) -> List[int]:
    """Random document lengths for small fuzz cases (1-token and empty documents included)."""
    out: List[int] = []
    s = 0
    while s < total:
        r = rng.random()
        if r < p_empty:
            length = 0
        elif r < p_empty + p_one:
            length = 1
        else:
            length = int(rng.integers(2, max_len + 1))
        length = min(length, total - s)
        out.append(length)
        s += length
    return out

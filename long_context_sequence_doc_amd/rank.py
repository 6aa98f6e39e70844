"""One sequence-parallel rank's forward: its ring steps issued through the C ABI.

The SP blog page (bmjup.com/post/14448.html, core principles) describes the
ring: each GPU holds one token chunk of Q and the KV chunks pass round the
ring, so after P steps every rank holds the full-sequence result for its
rows. Here the KV chunks of every step are already resident (they are views
into whole-sequence K/V buffers, selected by each step's segment table), and
one rank's work is:

    step 0 (the rank's own chunks; every local row sees at least itself):
        sap_attn_fwd -> running O / LSE
    each later step whose plan lists any tile:
        sap_attn_fwd_merge -> its partial merged into the running O / LSE in
        the kernel epilogue (touched rows with a key only; the others are
        exact as they are)
      or, with fused_merge=False, the two-pass form:
        sap_attn_fwd -> partial O / LSE of the touched rows
        sap_lse_merge   (touched rows only)
    steps with no tile launch nothing -- the sequence-aware part: with
    document masks most remote chunks of a rank hold no key its rows may see.

A head-sharded (Ulysses) rank is the one-step case with Q = KV = the whole
sequence for its heads. A rank that already holds every step's KV can also
run all steps as one call: ``concatenated(...)`` builds one plan over the
union of the steps' KV segments (one launch, no merge at all).

The backward (RankBackward) runs the recompute-based backward once per
non-empty step with the final O and LSE; the per-step dQ / dK / dV add up to
the full gradient.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import torch

from . import (sap_attn_bwd_accumulate, sap_attn_bwd_dkdv, sap_attn_bwd_dq, sap_attn_bwd_rowterm,
               sap_attn_bwd_workspace, sap_attn_fwd, sap_attn_fwd_merge, sap_lse_merge, sap_plan, sap_plan_free,
               sap_plan_info, sap_plan_q_tiles, sap_plan_upload)

BLOCK_M, BLOCK_N = 128, 64
N_CU = 256


def forward_block_m(q_segs, hq: int, hkv: int) -> int:
    """Q tile height of the forward plans: 256 when the GQA group is odd (a
    workgroup then holds one head, and 256-row tiles let 8 waves share each
    staged K / V tile, in the software-pipelined loop, instead of 4 in the
    plain one) and the rank has rows enough for about four such workgroups
    per compute unit (the 64K, 5-head shard is 4 % faster with 256 rows, the
    512K, 4-head one 6 %; the 32K, 32-head ring rank, with two per compute
    unit, 5 % slower); else 128 (even groups pair two heads per workgroup
    instead)."""
    tq = max(ls + ge - gs for gs, ge, ls in q_segs)
    if (hq // hkv) % 2 == 1 and (tq // 256) * hq >= 4 * N_CU:
        return 256
    return BLOCK_M


class RankForward:
    def __init__(self, cu_seqlens, q_segs: Sequence[Tuple[int, int, int]],
                 step_kv_segs: List[Sequence[Tuple[int, int, int]]], hq: int, hkv: int, d: int,
                 scale: float, device: str = "cuda", fused_merge: bool = True, block_m: int = 0):
        self.hq, self.hkv, self.d, self.scale = hq, hkv, d, scale
        self.fused_merge = fused_merge
        self.block_m = block_m or forward_block_m(q_segs, hq, hkv)
        self.plans = [sap_plan(cu_seqlens, q_segs, kv, self.block_m, BLOCK_N) for kv in step_kv_segs]
        self.infos = [sap_plan_info(p) for p in self.plans]
        first = self.infos[0]
        if first["n_touched_q_tiles"] != first["n_q_tiles"]:
            raise ValueError("step 0 must hold the rank's own chunks (it has to touch every local Q tile)")
        self.tq = first["tq"]
        self.active = [i for i, inf in enumerate(self.infos) if inf["n_tiles"] > 0]
        for i in self.active:
            sap_plan_upload(self.plans[i])
        self.o = torch.empty((self.tq, hq, d), dtype=torch.float32, device=device)
        self.lse = torch.empty((hq, self.tq), dtype=torch.float32, device=device)
        need_part = len(self.active) > 1 and not fused_merge
        self.o_part = torch.empty_like(self.o) if need_part else None
        self.lse_part = torch.empty_like(self.lse) if need_part else None

    @property
    def useful_pairs_per_head(self) -> int:
        return sum(inf["useful_pairs_per_head"] for inf in self.infos)

    @property
    def useful_flop(self) -> float:
        """Forward FLOP counted on allowed (query, key) pairs only: 4 D per pair per query head."""
        return 4.0 * self.d * self.hq * self.useful_pairs_per_head

    def merge_rows(self) -> int:
        """(row, head) pairs merged per run (touched rows of every step after the first)."""
        rows = 0
        for i in self.active[1:]:
            touched, desc = sap_plan_q_tiles(self.plans[i])
            rows += int(desc[touched, 1].sum())
        return rows * self.hq

    def touched_rows(self, step: int):
        """Local Q rows the given step's forward writes."""
        touched, desc = sap_plan_q_tiles(self.plans[step])
        return [r for t in touched for r in range(desc[t, 0], desc[t, 0] + desc[t, 1])]

    def run(self, q, k, v, q_row_stride: int, kv_row_stride: int, stream=None):
        """q: local Q rows [tq, hq, d] bf16; k, v: buffers addressed by the steps' local rows."""
        for n, i in enumerate(self.active):
            p = self.plans[i]
            if n == 0:
                sap_attn_fwd(p, q, k, v, q_row_stride, kv_row_stride, self.hq, self.hkv, self.d, self.scale,
                             self.o, self.lse, stream)
            elif self.fused_merge:
                sap_attn_fwd_merge(p, q, k, v, q_row_stride, kv_row_stride, self.hq, self.hkv, self.d, self.scale,
                                   self.o, self.lse, stream)
            else:
                sap_attn_fwd(p, q, k, v, q_row_stride, kv_row_stride, self.hq, self.hkv, self.d, self.scale,
                             self.o_part, self.lse_part, stream)
                sap_lse_merge(p, self.o, self.lse, self.o_part, self.lse_part, self.tq, self.hq, self.d, stream)
        return self.o, self.lse

    def close(self):
        for p in self.plans:
            sap_plan_free(p)
        self.plans = []

    @classmethod
    def local_then_remote(cls, cu_seqlens, q_segs, step_kv_segs, hq: int, hkv: int, d: int, scale: float,
                          device: str = "cuda", block_m: int = 0):
        """Two calls: the rank's own chunks (step 0), then one merged call over
        the KV of every later step together -- the schedule of a rank that
        fetches all the remote chunks its plan needs at once (from their
        owners, in parallel) while it computes on its own chunks."""
        remote = [seg for segs in step_kv_segs[1:] for seg in segs]
        return cls(cu_seqlens, q_segs, [step_kv_segs[0], remote], hq, hkv, d, scale, device, block_m=block_m)

    @classmethod
    def concatenated(cls, cu_seqlens, q_segs, step_kv_segs, hq: int, hkv: int, d: int, scale: float,
                     device: str = "cuda", block_m: int = 0):
        """One forward call over every step's KV segments together (the steps
        must address disjoint KV rows): the fused ring pass for a rank whose KV
        chunks are all resident."""
        union = [seg for segs in step_kv_segs for seg in segs]
        return cls(cu_seqlens, q_segs, [union], hq, hkv, d, scale, device, block_m=block_m)


class RankBackward:
    """The rank's backward, given the final (merged) O and LSE:
        sap_attn_bwd_rowterm once, with the plan of the rank's own chunk (it
        touches every local row): D_r = dO_r . O_r;
        sap_attn_bwd_accumulate per non-empty ring step, adding that step's
        share into the caller's dq / dk / dv (zeroed by the caller once per
        training step); the shares sum to the full gradient. The steps run in
        order on one stream and share one workspace (partial sums of split
        KV tiles)."""

    BLOCK_M, BLOCK_N = 64, 128

    def __init__(self, cu_seqlens, q_segs: Sequence[Tuple[int, int, int]],
                 step_kv_segs: List[Sequence[Tuple[int, int, int]]], hq: int, hkv: int, d: int,
                 scale: float, device: str = "cuda"):
        self.hq, self.hkv, self.d, self.scale = hq, hkv, d, scale
        self.plans = [sap_plan(cu_seqlens, q_segs, kv, self.BLOCK_M, self.BLOCK_N) for kv in step_kv_segs]
        self.infos = [sap_plan_info(p) for p in self.plans]
        first = self.infos[0]
        if first["n_touched_q_tiles"] != first["n_q_tiles"]:
            raise ValueError("step 0 must hold the rank's own chunks (it has to touch every local Q tile)")
        self.tq = first["tq"]
        self.active = [i for i, inf in enumerate(self.infos) if inf["n_tiles"] > 0]
        for i in self.active:
            sap_plan_upload(self.plans[i])
        self.delta = torch.empty((hq, max(self.tq, 1)), dtype=torch.float32, device=device)
        self.ws_bytes = max([sap_attn_bwd_workspace(self.plans[i], 0, hkv, d) for i in self.active] + [0])
        self.ws = torch.empty(max(self.ws_bytes // 4, 4), dtype=torch.float32, device=device)

    @property
    def useful_pairs_per_head(self) -> int:
        return sum(inf["useful_pairs_per_head"] for inf in self.infos)

    @property
    def useful_flop(self) -> float:
        """Backward FLOP on allowed pairs: 10 D per pair per query head (recompute of
        Q K^T and dO V^T, then dV, dK, dQ)."""
        return 10.0 * self.d * self.hq * self.useful_pairs_per_head

    def rowterm(self, o, dout, q_row_stride: int, stream=None):
        sap_attn_bwd_rowterm(self.plans[0], o, dout, q_row_stride, self.hq, self.d, self.delta, stream)

    def accumulate(self, i: int, q, k, v, lse, dout, q_row_stride: int, kv_row_stride: int, dq, dk, dv,
                   stream=None):
        sap_attn_bwd_accumulate(self.plans[i], q, k, v, lse, self.delta, dout, q_row_stride, kv_row_stride,
                                self.hq, self.hkv, self.d, self.scale, dq, dk, dv, self.ws, self.ws_bytes, stream)

    def dkdv(self, i: int, q, k, v, lse, dout, q_row_stride: int, kv_row_stride: int, dk, dv, stream=None):
        """Step i's dK / dV pass alone (the first half of ``accumulate``)."""
        sap_attn_bwd_dkdv(self.plans[i], q, k, v, lse, self.delta, dout, q_row_stride, kv_row_stride, self.hq,
                          self.hkv, self.d, self.scale, dk, dv, self.ws, self.ws_bytes, stream)

    def dq(self, i: int, q, k, v, lse, dout, q_row_stride: int, kv_row_stride: int, dq, stream=None):
        """Step i's dQ pass alone (the second half of ``accumulate``)."""
        sap_attn_bwd_dq(self.plans[i], q, k, v, lse, self.delta, dout, q_row_stride, kv_row_stride, self.hq,
                        self.hkv, self.d, self.scale, dq, stream)

    def run(self, q, k, v, o, lse, dout, q_row_stride: int, kv_row_stride: int, dq, dk, dv, stream=None):
        self.rowterm(o, dout, q_row_stride, stream)
        for i in self.active:
            self.accumulate(i, q, k, v, lse, dout, q_row_stride, kv_row_stride, dq, dk, dv, stream)

    def close(self):
        for p in self.plans:
            sap_plan_free(p)
        self.plans = []

    @classmethod
    def local_then_remote(cls, cu_seqlens, q_segs, step_kv_segs, hq: int, hkv: int, d: int, scale: float,
                          device: str = "cuda"):
        """Two accumulate calls: the rank's own chunks, then every later step's
        KV together (the backward of RankForward.local_then_remote)."""
        remote = [seg for segs in step_kv_segs[1:] for seg in segs]
        return cls(cu_seqlens, q_segs, [step_kv_segs[0], remote], hq, hkv, d, scale, device)

    @classmethod
    def concatenated(cls, cu_seqlens, q_segs, step_kv_segs, hq: int, hkv: int, d: int, scale: float,
                     device: str = "cuda"):
        """The backward of every step's KV segments as one call (the steps must
        address disjoint KV rows): one dK/dV pass and one dQ pass for a rank
        whose KV chunks are all resident."""
        union = [seg for segs in step_kv_segs for seg in segs]
        return cls(cu_seqlens, q_segs, [union], hq, hkv, d, scale, device)

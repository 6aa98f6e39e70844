"""GPU parity of the backward (bwd_preprocess + attn_bwd) against the fp64 oracle.

The backward consumes the final O and LSE; the small cases feed the GPU the
oracle's O / LSE (rounded to fp32) to test the backward in isolation, the
full-size training case the GPU forward's (as a training step would) while
the oracle runs its own forward. dQ / dK / dV
are compared max-abs within 2e-2 (bf16 inputs; P and dS rounded to bf16 for
the matrix cores; fp32 accumulation). Every call goes through the C ABI.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from tests.gpu_common import TOL_O, f64, full_reference, need_gpu, say, tensors, to_dev

pytestmark = pytest.mark.gpu


def _sap():
    need_gpu()
    import long_context_sequence_doc_amd as sap
    return sap


def _globals(segs, n):
    g = np.full(n, -1, dtype=np.int64)
    for gs, ge, ls in segs:
        g[ls:ls + ge - gs] = np.arange(gs, ge)
    return g


def _check(name, got, ref, rows=None):
    got = np.asarray(got, dtype=np.float64)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert not np.isnan(got).any(), f"{name}: NaN"
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    say(f"  {name}: max|err|={err:.3e} (max|ref|={np.abs(ref).max():.2e})")
    assert err <= TOL_O, f"{name}: {err}"


def _bwd_call(sap, cu, q_segs, kv_segs, qd, kd, vd, dod, o, lse, hq, hkv, d, scale, dq, dk, dv):
    import torch
    plan = sap.sap_plan(cu, q_segs, kv_segs, 64, 128)
    info = sap.sap_plan_info(plan)
    if info["n_tiles"]:
        sap.sap_plan_upload(plan)
    ws_bytes = sap.sap_attn_bwd_workspace(plan, hq, hkv, d)
    ws = torch.empty(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")
    sap.sap_attn_bwd(plan, qd, kd, vd, o, lse, dod, qd.stride(0), kd.stride(0), hq, hkv, d, scale,
                     dq, dk, dv, ws, ws.numel() * 4)
    return plan, ws          # the caller keeps both alive until the stream is synchronised


@pytest.mark.parametrize("seed", range(10))
def test_random_small_layouts(seed):
    """Ragged tiles, 1-token and empty documents, GQA (group sizes 1-4; odd
    and even groups take different workgroup shapes), D in {64, 128}, a
    sharded Q (two segments, local != global rows), KV in two pieces and, on
    odd seeds, K / V rows strided past their heads."""
    sap = _sap()
    import torch
    rng = np.random.default_rng(700 + seed)
    d = 128 if seed % 2 else 64
    hkv = int(rng.choice([1, 2]))
    hq = hkv * (int(rng.choice([1, 2, 4])) if seed < 8 else 3)
    total = int(rng.integers(200, 900))
    lengths = W.random_docs(rng, total, int(rng.integers(2, 400)))
    cu = W.cu_seqlens(lengths)
    a = int(rng.integers(0, total - 1))
    q_segs = [(a, total, 5), (0, a, total - a + 9)] if a > 0 else [(0, total, 0)]
    c0 = int(rng.integers(0, total))
    kv_segs = [(c0, total, 0), (0, c0, total - c0 + 3)] if c0 > 0 else [(0, total, 0)]
    say(f"case bwd random seed={seed} total={total} docs={len(lengths)} hq={hq} hkv={hkv} d={d}")
    scale = 1.0 / np.sqrt(d)
    gq = _globals(q_segs, max(ls + ge - gs for gs, ge, ls in q_segs))
    gk = _globals(kv_segs, max(ls + ge - gs for gs, ge, ls in kv_segs))
    rs = np.random.default_rng(seed)
    mk = lambda h: W.bf16_round(rs.standard_normal((total, h, d), dtype=np.float32))
    qf, kf, vf, dof = mk(hq), mk(hkv), mk(hkv), mk(hq)
    ql = np.zeros((len(gq), hq, d), dtype=np.uint16)
    dol = np.zeros((len(gq), hq, d), dtype=np.uint16)
    # K / V rows padded by an extra head on odd seeds (kv_row_stride > hkv * d)
    kpad = hkv + (seed % 2)
    kl = np.zeros((len(gk), kpad, d), dtype=np.uint16)
    vl = np.zeros((len(gk), kpad, d), dtype=np.uint16)
    vq, vk = gq >= 0, gk >= 0
    ql[vq], dol[vq] = qf[gq[vq]], dof[gq[vq]]
    kl[vk, :hkv], vl[vk, :hkv] = kf[gk[vk]], vf[gk[vk]]
    gq0 = np.where(vq, gq, 0)
    gk0 = np.where(vk, gk, -10 ** 9)
    k64, v64 = f64(kl[:, :hkv]), f64(vl[:, :hkv])
    # final O / LSE from the oracle over this call's KV (= all keys here)
    o_ref, lse_ref = A.forward(f64(ql), k64, v64, gq0, gk0, cu, scale)
    rows = np.nonzero(vq)[0]
    dq_ref, dk_ref, dv_ref = A.backward(f64(ql), k64, v64, f64(dol), o_ref, lse_ref, gq0, gk0, cu, scale)
    qd, kd, vd, dod = to_dev(ql), to_dev(kl), to_dev(vl), to_dev(dol)
    o = torch.from_numpy(o_ref.astype(np.float32)).cuda()
    lse = torch.from_numpy(lse_ref.astype(np.float32)).cuda()
    dq = torch.zeros((len(gq), hq, d), device="cuda")
    dk = torch.zeros((len(gk), hkv, d), device="cuda")
    dv = torch.zeros((len(gk), hkv, d), device="cuda")
    keep = _bwd_call(sap, cu, q_segs, kv_segs, qd, kd, vd, dod, o, lse, hq, hkv, d, scale, dq, dk, dv)
    torch.cuda.synchronize()
    del keep                                      # plans are freed only after the kernels finished
    _check("dQ", dq.cpu().numpy(), dq_ref, rows)
    kr = np.nonzero(vk)[0]
    _check("dK", dk.cpu().numpy(), dk_ref, kr)
    _check("dV", dv.cpu().numpy(), dv_ref, kr)
    # rows outside every segment were never touched
    assert (dq.cpu().numpy()[~vq] == 0).all() and (dk.cpu().numpy()[~vk] == 0).all()


@pytest.mark.parametrize("case", [(2, 1, 128, [4096]), (1, 1, 64, [3000, 1096]), (4, 2, 128, [1500, 2596]),
                                  (8, 2, 64, [2500, 1, 1595]), (4, 1, 64, [4096])])
def test_split_kv_tiles_all_rows(case):
    """Documents long enough that KV tiles meet more partner Q tiles than one
    workgroup takes: their chunks leave partial sums in workspace slots and
    the ordered reduce adds them. Every dQ, dK, dV row against the oracle.
    GQA groups of 1, 2 and 4 at both head dims between them, so every
    compiled dQ workgroup shape (one, two and four query heads) and both
    dK / dV kernels run."""
    sap = _sap()
    import torch
    hq, hkv, d, lengths = case
    cu = W.cu_seqlens(lengths)
    total = int(cu[-1])
    scale = 1.0 / np.sqrt(d)
    say(f"case bwd split tiles hq={hq} hkv={hkv} d={d} docs={lengths}")
    rs = np.random.default_rng(40 + hq + d)
    mk = lambda h: W.bf16_round(rs.standard_normal((total, h, d), dtype=np.float32))
    qb, kb, vb, dob = mk(hq), mk(hkv), mk(hkv), mk(hq)
    g = np.arange(total)
    o_ref, lse_ref = A.forward(f64(qb), f64(kb), f64(vb), g, g, cu, scale)
    dq_ref, dk_ref, dv_ref = A.backward(f64(qb), f64(kb), f64(vb), f64(dob), o_ref, lse_ref, g, g, cu, scale)
    segs = [(0, total, 0)]
    plan = sap.sap_plan(cu, segs, segs, 64, 128)
    # the plan must split some KV tile: workspace beyond the row terms
    assert sap.sap_attn_bwd_workspace(plan, hq, hkv, d) > hq * total * 4 + 256
    sap.sap_plan_free(plan)
    qd, kd, vd, dod = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(dob)
    o = torch.from_numpy(o_ref.astype(np.float32)).cuda()
    lse = torch.from_numpy(lse_ref.astype(np.float32)).cuda()
    dq = torch.zeros((total, hq, d), device="cuda")
    dk = torch.zeros((total, hkv, d), device="cuda")
    dv = torch.zeros((total, hkv, d), device="cuda")
    keep = _bwd_call(sap, cu, segs, segs, qd, kd, vd, dod, o, lse, hq, hkv, d, scale, dq, dk, dv)
    torch.cuda.synchronize()
    del keep
    _check("dQ split", dq.cpu().numpy(), dq_ref)
    _check("dK split", dk.cpu().numpy(), dk_ref)
    _check("dV split", dv.cpu().numpy(), dv_ref)


@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 128), (8, 2, 64)])
def test_backward_is_deterministic_and_halves_compose(hq, hkv, d):
    """sap_attn_bwd twice into zeroed buffers on a plan that splits KV tiles:
    bit-identical dQ, dK, dV (the split tiles' slots are added in a fixed
    order, no atomics). Then the parts -- sap_attn_bwd_rowterm,
    sap_attn_bwd_dkdv, sap_attn_bwd_dq -- give the same bits as the one call,
    and sap_attn_bwd_dkdv leaves dQ alone, sap_attn_bwd_dq dK / dV."""
    sap = _sap()
    import torch
    lengths = [3000, 7, 1089]
    cu = W.cu_seqlens(lengths)
    total = int(cu[-1])
    scale = 1.0 / np.sqrt(d)
    say(f"case bwd determinism hq={hq} hkv={hkv} d={d} docs={lengths}")
    rs = np.random.default_rng(61 + d)
    mk = lambda h: W.bf16_round(rs.standard_normal((total, h, d), dtype=np.float32))
    qb, kb, vb, dob = mk(hq), mk(hkv), mk(hkv), mk(hq)
    segs = [(0, total, 0)]
    plan = sap.sap_plan(cu, segs, segs, 64, 128)
    sap.sap_plan_upload(plan)
    ws_all = sap.sap_attn_bwd_workspace(plan, hq, hkv, d)
    ws_kv = sap.sap_attn_bwd_workspace(plan, 0, hkv, d)
    assert ws_kv > 0, "the plan must split some KV tile"
    qd, kd, vd, dod = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(dob)
    # the final O / LSE from the GPU forward (a training step's inputs)
    fplan = sap.sap_plan(cu, segs, segs, 128, 64)
    sap.sap_plan_upload(fplan)
    o = torch.empty((total, hq, d), device="cuda")
    lse = torch.empty((hq, total), device="cuda")
    sap.sap_attn_fwd(fplan, qd, kd, vd, qd.stride(0), kd.stride(0), hq, hkv, d, scale, o, lse)
    ws = torch.empty(ws_all // 4 + 64, dtype=torch.float32, device="cuda")
    outs = []
    for rep in range(2):
        dq = torch.zeros((total, hq, d), device="cuda")
        dk = torch.zeros((total, hkv, d), device="cuda")
        dv = torch.zeros((total, hkv, d), device="cuda")
        ws.fill_(float("nan") if rep else 7.0)   # workspace contents on entry do not matter
        sap.sap_attn_bwd(plan, qd, kd, vd, o, lse, dod, qd.stride(0), kd.stride(0), hq, hkv, d, scale, dq, dk, dv,
                         ws, ws.numel() * 4)
        torch.cuda.synchronize()
        outs.append((dq, dk, dv))
    for a, b, name in zip(outs[0], outs[1], ("dQ", "dK", "dV")):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{name} differs between two runs"
    # the parts, into fresh zeroed buffers
    delta = torch.empty((hq, total), device="cuda")
    dq = torch.zeros((total, hq, d), device="cuda")
    dk = torch.zeros((total, hkv, d), device="cuda")
    dv = torch.zeros((total, hkv, d), device="cuda")
    part = torch.empty(ws_kv // 4 + 64, dtype=torch.float32, device="cuda")
    sap.sap_attn_bwd_rowterm(plan, o, dod, dod.stride(0), hq, d, delta)
    sap.sap_attn_bwd_dkdv(plan, qd, kd, vd, lse, delta, dod, qd.stride(0), kd.stride(0), hq, hkv, d, scale, dk, dv,
                          part, part.numel() * 4)
    torch.cuda.synchronize()
    assert not dq.any(), "the dK/dV pass wrote dQ"
    sap.sap_attn_bwd_dq(plan, qd, kd, vd, lse, delta, dod, qd.stride(0), kd.stride(0), hq, hkv, d, scale, dq)
    torch.cuda.synchronize()
    for a, b, name in zip(outs[0], (dq, dk, dv), ("dQ", "dK", "dV")):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{name}: parts differ from the one call"
    # and the values against the oracle (every row)
    g = np.arange(total)
    o_ref, lse_ref = A.forward(f64(qb), f64(kb), f64(vb), g, g, cu, scale)
    dq_ref, dk_ref, dv_ref = A.backward(f64(qb), f64(kb), f64(vb), f64(dob), o_ref, lse_ref, g, g, cu, scale)
    _check("dQ det", dq.cpu().numpy(), dq_ref)
    _check("dK det", dk.cpu().numpy(), dk_ref)
    _check("dV det", dv.cpu().numpy(), dv_ref)
    sap.sap_plan_free(plan)
    sap.sap_plan_free(fplan)


@pytest.mark.parametrize("group,hkv,d,seed", [(8, 1, 128, 0), (8, 2, 64, 1), (6, 1, 128, 2), (5, 2, 128, 3),
                                               (5, 1, 64, 4)])
def test_wide_gqa_groups_fwd_bwd_all_rows(group, hkv, d, seed):
    """GQA groups beyond the workloads' 1-4 (5 and 6: odd / even head
    pairing; 8: four head pairs per KV head in the forward and two four-head
    dQ workgroups per KV head in the backward) on a random layout with long
    and 1-token documents: the forward through the C ABI against the oracle on
    every row, then the backward from the GPU's own O / LSE (a training step's
    data flow) on every dQ row and dK / dV key. dK / dV of a KV head sum over
    the group's query heads, so the bf16 rounding of P and dS grows with the
    group; the 2e-2 bound still holds at 8 (group 16 reaches 2.7e-2 on dV,
    1.5e-3 of its largest value)."""
    sap = _sap()
    import torch
    hq = group * hkv
    rng = np.random.default_rng(4400 + seed)
    total = int(rng.integers(700, 1300))
    lengths = W.random_docs(rng, total, int(rng.integers(200, 900)))
    cu = W.cu_seqlens(lengths)
    say(f"case wide GQA group={group} hq={hq} hkv={hkv} d={d} total={total} docs={len(lengths)}")
    scale = 1.0 / np.sqrt(d)
    rs = np.random.default_rng(seed)
    mk = lambda h: W.bf16_round(rs.standard_normal((total, h, d), dtype=np.float32))
    qf, kf, vf, dof = mk(hq), mk(hkv), mk(hkv), mk(hq)
    pos = np.arange(total)
    o_ref, lse_ref = A.forward(f64(qf), f64(kf), f64(vf), pos, pos, cu, scale)
    dq_ref, dk_ref, dv_ref = A.backward(f64(qf), f64(kf), f64(vf), f64(dof), o_ref, lse_ref, pos, pos, cu, scale)
    seg = [(0, total, 0)]
    qd, kd, vd, dod = to_dev(qf), to_dev(kf), to_dev(vf), to_dev(dof)
    plan = sap.sap_plan(cu, seg, seg, 128, 64)
    sap.sap_plan_upload(plan)
    o = torch.full((total, hq, d), float("nan"), device="cuda")
    lse = torch.full((hq, total), float("nan"), device="cuda")
    sap.sap_attn_fwd(plan, qd, kd, vd, qd.stride(0), kd.stride(0), hq, hkv, d, scale, o, lse)
    torch.cuda.synchronize()
    o_h, lse_h = o.cpu().numpy(), lse.cpu().numpy()
    eo = float(np.abs(o_h - o_ref).max())
    el = float(np.abs(lse_h - lse_ref).max())
    say(f"  forward: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= 1e-3
    dq = torch.zeros((total, hq, d), device="cuda")
    dk = torch.zeros((total, hkv, d), device="cuda")
    dv = torch.zeros((total, hkv, d), device="cuda")
    keep = _bwd_call(sap, cu, seg, seg, qd, kd, vd, dod, o, lse, hq, hkv, d, scale, dq, dk, dv)
    torch.cuda.synchronize()
    del keep, plan
    _check("dQ", dq.cpu().numpy(), dq_ref)
    _check("dK", dk.cpu().numpy(), dk_ref)
    _check("dV", dv.cpu().numpy(), dv_ref)


def test_ring_steps_accumulate_to_full_gradient():
    """Per-step calls with the final LSE add up (dq/dk/dv are accumulated)."""
    sap = _sap()
    import torch
    rng = np.random.default_rng(11)
    total, hq, hkv, d = 768, 4, 2, 128
    lengths = W.random_docs(rng, total, 300)
    cu = W.cu_seqlens(lengths)
    scale = 1.0 / np.sqrt(d)
    mk = lambda h: W.bf16_round(rng.standard_normal((total, h, d), dtype=np.float32))
    qf, kf, vf, dof = mk(hq), mk(hkv), mk(hkv), mk(hq)
    g = np.arange(total)
    q_segs = [(256, 512, 0)]                      # the rank's rows
    gq = np.arange(256, 512)
    o_ref, lse_ref = A.forward(f64(qf[256:512]), f64(kf), f64(vf), gq, g, cu, scale)
    dq_ref, dk_ref, dv_ref = A.backward(f64(qf[256:512]), f64(kf), f64(vf), f64(dof[256:512]), o_ref, lse_ref,
                                        gq, g, cu, scale)
    qd, dod = to_dev(qf[256:512]), to_dev(dof[256:512])
    kd, vd = to_dev(kf), to_dev(vf)
    o = torch.from_numpy(o_ref.astype(np.float32)).cuda()
    lse = torch.from_numpy(lse_ref.astype(np.float32)).cuda()
    dq = torch.zeros((256, hq, d), device="cuda")
    dk = torch.zeros((total, hkv, d), device="cuda")
    dv = torch.zeros((total, hkv, d), device="cuda")
    say("case bwd ring: 3 KV chunks of 256, accumulated")
    keep = []
    for c in range(3):
        keep.append(_bwd_call(sap, cu, q_segs, [(256 * c, 256 * (c + 1), 256 * c)], qd, kd, vd, dod, o, lse,
                              hq, hkv, d, scale, dq, dk, dv))
    torch.cuda.synchronize()
    del keep
    _check("dQ ring", dq.cpu().numpy(), dq_ref)
    _check("dK ring", dk.cpu().numpy(), dk_ref)
    _check("dV ring", dv.cpu().numpy(), dv_ref)
    # the same three chunks as one plan and one call
    say("case bwd ring: the 3 KV chunks in one call")
    dq.zero_(); dk.zero_(); dv.zero_()
    keep = _bwd_call(sap, cu, q_segs, [(256 * c, 256 * (c + 1), 256 * c) for c in range(3)], qd, kd, vd, dod, o,
                     lse, hq, hkv, d, scale, dq, dk, dv)
    torch.cuda.synchronize()
    del keep
    _check("dQ one call", dq.cpu().numpy(), dq_ref)
    _check("dK one call", dk.cpu().numpy(), dk_ref)
    _check("dV one call", dv.cpu().numpy(), dv_ref)


def test_training_fwd_bwd_all_rows():
    """64K training sequence (5 heads, 30 documents incl. 1-token ones):
    GPU forward then GPU backward; every dQ row and every dK / dV key against
    the oracle (which runs its own forward for the final O / LSE)."""
    sap = _sap()
    import torch
    from long_context_sequence_doc_amd.rank import RankForward
    w = W.training()
    t = tensors("train", True)
    say("case train_64k_5heads fwd+bwd, every row and key")
    rf = RankForward(w.cu, w.q_segs, [s.kv_segs for s in w.steps], w.hq, w.hkv, w.d, w.scale)
    qd, kd, vd, dod = to_dev(t.q), to_dev(t.k), to_dev(t.v), to_dev(t.do)
    o, lse = rf.run(qd, kd, vd, qd.stride(0), kd.stride(0))
    dq = torch.zeros((w.total, w.hq, w.d), device="cuda")
    dk = torch.zeros_like(dq)
    dv = torch.zeros_like(dq)
    keep = _bwd_call(sap, w.cu, w.q_segs, w.steps[0].kv_segs, qd, kd, vd, dod, o, lse, w.hq, w.hkv, w.d,
                     w.scale, dq, dk, dv)
    torch.cuda.synchronize()
    del keep
    dq_h, dk_h, dv_h = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    rf.close()
    _, _, dq_ref, dk_ref, dv_ref = full_reference("train")
    _check("dQ train (all rows)", dq_h, dq_ref)
    _check("dK train (all keys)", dk_h, dk_ref)
    _check("dV train (all keys)", dv_h, dv_ref)


def _heaviest_kv_tile_keys(rb, step_kv_segs):
    """Local rows of the split KV tile with the most partner Q tiles over the
    backward's plans, and that count. A split tile's dK / dV are partial sums
    in workspace slots that the ordered reduce adds up (the split rule is
    written out in tests/kv_chunks.py)."""
    from oracle import planner as PL
    from tests.kv_chunks import kv_chunks
    best, keys = -1, []
    for i in rb.active:
        for t, runs in kv_chunks(rb.plans[i]).items():
            if len(runs) > 1 and sum(runs) > best:
                ls, nr, _ = PL.tiles_of(step_kv_segs[i], 128)[t]
                best, keys = sum(runs), list(range(ls, ls + nr))
    assert best > 0, "no KV tile of the backward plans is split"
    return best, keys


def _rank_fwd_bwd_all_rows(w, ref, label, active, two_calls=False):
    """A 128K-sequence rank: forward with merges, row terms once, backward per
    non-empty step (or as own + remote calls); every dQ row and every dK / dV
    key of every head against the oracle's full reference ``ref``; the keys
    of the backward plans' heaviest (split) KV tile are reported on their own."""
    import torch
    from long_context_sequence_doc_amd.rank import RankBackward, RankForward
    t = tensors("zigzag", True)
    steps = [s.kv_segs for s in w.steps]
    if two_calls:
        rf = RankForward.local_then_remote(w.cu, w.q_segs, steps, w.hq, w.hkv, w.d, w.scale)
        rb = RankBackward.local_then_remote(w.cu, w.q_segs, steps, w.hq, w.hkv, w.d, w.scale)
        bwd_steps = [steps[0], [seg for segs in steps[1:] for seg in segs]]
    else:
        rf = RankForward(w.cu, w.q_segs, steps, w.hq, w.hkv, w.d, w.scale)
        rb = RankBackward(w.cu, w.q_segs, steps, w.hq, w.hkv, w.d, w.scale)
        bwd_steps = steps
    if active is not None:
        assert rb.active == active
    ql, dol = W.local_rows(t.q, w.q_segs), W.local_rows(t.do, w.q_segs)
    qd, dod, kd, vd = to_dev(ql), to_dev(dol), to_dev(t.k), to_dev(t.v)
    o, lse = rf.run(qd, kd, vd, qd.stride(0), kd.stride(0))
    dq = torch.zeros((w.tq, w.hq, w.d), device="cuda")
    dk = torch.zeros((w.total, w.hkv, w.d), device="cuda")
    dv = torch.zeros_like(dk)
    rb.run(qd, kd, vd, o, lse, dod, qd.stride(0), kd.stride(0), dq, dk, dv)
    torch.cuda.synchronize()
    heavy_n, heavy = _heaviest_kv_tile_keys(rb, bwd_steps)
    say(f"  heaviest KV tile of the backward plans: {heavy_n} partner Q tiles (split), keys {heavy[0]}..{heavy[-1]}")
    dq_h, dk_h, dv_h = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    rf.close()
    rb.close()
    _, _, dq_ref, dk_ref, dv_ref = full_reference(ref)
    _check(f"dQ {label} (all rows)", dq_h, dq_ref)
    _check(f"dK {label} (all keys)", dk_h, dk_ref)
    _check(f"dV {label} (all keys)", dv_h, dv_ref)
    _check(f"dK {label} (heaviest split KV tile)", dk_h[heavy], dk_ref[heavy])


def test_zigzag_rank_fwd_bwd_all_rows():
    """The benchmarked configuration: 128K zigzag GQA rank 3 (ring steps 0, 1, 7)."""
    _sap()
    say("case zigzag_sp8_128k_gqa_rank3 fwd+bwd (ring steps), every row and key")
    _rank_fwd_bwd_all_rows(W.zigzag_rank(3), "zigzag", "zigzag", active=[0, 1, 7])


def test_zigzag_rank_two_calls_all_rows():
    """128K zigzag GQA rank 3, forward and backward as two calls each (own
    chunks, then all remote chunks at once)."""
    _sap()
    say("case zigzag_sp8_128k_gqa_rank3 fwd+bwd as local + remote calls, every row and key")
    _rank_fwd_bwd_all_rows(W.zigzag_rank(3), "zigzag", "zigzag two calls", active=[0, 1], two_calls=True)


def test_balanced_rank_fwd_bwd_all_rows():
    """The same 128K sequence in the document-aware balanced layout (1024-row
    chunks from sap_balance), rank 3: scattered Q chunks, all 8 ring steps;
    every row and key."""
    sap = _sap()
    from oracle import balance as B
    z = W.zigzag_rank(3)
    owner, _ = sap.sap_balance(z.cu, 8, 1024)
    assert owner.tolist() == B.balance(z.cu, 8, 1024)[0]
    w = W.owner_rank(z, owner.tolist(), 3, 1024, "balanced")
    say(f"case balanced_sp8_128k_gqa_rank3 fwd+bwd ({len(w.q_segs)} Q segments), every row and key")
    _rank_fwd_bwd_all_rows(w, "balanced", "balanced", active=None)


def test_plans_without_pairs_launch_nothing():
    """A call whose KV rows all lie after its queries (one document) has no
    allowed pair: every entry point returns OK and leaves its outputs
    bit-identical (poisoned buffers stay as they were), with or without an
    uploaded plan, and the stream stays usable."""
    sap = _sap()
    import torch
    say("case no allowed pair: Q rows [0, 256), KV rows [256, 512) of one 512-token document")
    hq, hkv, d, total = 4, 2, 128, 512
    cu = [0, total]
    for bm, bn in ((128, 64), (64, 128)):
        plan = sap.sap_plan(cu, [(0, 256, 0)], [(256, total, 0)], bm, bn)
        info = sap.sap_plan_info(plan)
        assert info["n_tiles"] == 0 and info["useful_pairs_per_head"] == 0
        q = torch.randn((256, hq, d), device="cuda").to(torch.bfloat16)
        kv = torch.randn((256, hkv, d), device="cuda").to(torch.bfloat16)
        o = torch.full((256, hq, d), float("nan"), device="cuda")
        lse = torch.full((hq, 256), 7.0, device="cuda")
        dq = torch.full((256, hq, d), 3.0, device="cuda")
        dk = torch.full((256, hkv, d), -2.0, device="cuda")
        dv = torch.full((256, hkv, d), 5.0, device="cuda")
        delta = torch.full((hq, 256), 11.0, device="cuda")
        before = [t.clone() for t in (o, lse, dq, dk, dv, delta)]
        if bm == 128:
            sap.sap_attn_fwd(plan, q, kv, kv, q.stride(0), kv.stride(0), hq, hkv, d, 0.088, o, lse)
            sap.sap_attn_fwd_merge(plan, q, kv, kv, q.stride(0), kv.stride(0), hq, hkv, d, 0.088, o, lse)
            sap.sap_lse_merge(plan, o, lse, o, lse, 256, hq, d)
        else:
            # the row terms still take hq x tq floats; no KV tile, so no partial-sum slots
            assert sap.sap_attn_bwd_workspace(plan, hq, hkv, d) == hq * 256 * 4
            assert sap.sap_attn_bwd_workspace(plan, 0, hkv, d) == 0
            sap.sap_attn_bwd_rowterm(plan, o, q, q.stride(0), hq, d, delta)
            sap.sap_attn_bwd_accumulate(plan, q, kv, kv, lse, delta, q, q.stride(0), kv.stride(0), hq, hkv, d,
                                        0.088, dq, dk, dv)
        torch.cuda.synchronize()
        for a, b in zip((o, lse, dq, dk, dv, delta), before):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        sap.sap_plan_free(plan)
    # the stream still runs work afterwards
    x = torch.ones(1024, device="cuda")
    assert float((x * 2).sum()) == 2048.0

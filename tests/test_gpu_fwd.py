"""GPU parity of the forward kernel and the merge against the fp64 oracle.

Every call goes through the C ABI (libsap.so). Tolerances: max-abs 2e-2 on
O, 1e-3 on finite LSE, -inf LSE matched exactly; the kernels see bf16 inputs
and the oracle the same values widened to fp64.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from tests.gpu_common import (TOL_LSE, TOL_O, compare, f64, full_reference, need_gpu, oracle_forward_rows,
                               sample_rows, say, tensors, to_dev, ulysses_rows)

pytestmark = pytest.mark.gpu


def _sap():
    need_gpu()
    import long_context_sequence_doc_amd as sap
    return sap


def _run_single(sap, cu, q_segs, kv_segs, q_bits, k_bits, v_bits, hq, hkv, d, scale, poison=True):
    """One sap_attn_fwd call; q_bits are local Q rows, k/v_bits local KV rows."""
    import torch
    plan = sap.sap_plan(cu, q_segs, kv_segs, 128, 64)
    info = sap.sap_plan_info(plan)
    tq = info["tq"]
    q = to_dev(q_bits)
    k = to_dev(k_bits)
    v = to_dev(v_bits)
    o = torch.full((tq, hq, d), float("nan") if poison else 0.0, device="cuda")
    lse = torch.full((hq, tq), float("nan") if poison else 0.0, device="cuda")
    if info["n_tiles"]:
        sap.sap_plan_upload(plan)
    sap.sap_attn_fwd(plan, q, k, v, q.stride(0), k.stride(0), hq, hkv, d, scale, o, lse)
    torch.cuda.synchronize()
    touched, desc = sap.sap_plan_q_tiles(plan)
    rows = np.array([r for t in touched for r in range(desc[t, 0], desc[t, 0] + desc[t, 1])], dtype=np.int64)
    return o.cpu().numpy(), lse.cpu().numpy(), rows, info


def _globals(segs, n):
    g = np.full(n, -1, dtype=np.int64)
    for gs, ge, ls in segs:
        g[ls:ls + ge - gs] = np.arange(gs, ge)
    return g


def test_tiny_full_sequence():
    sap = _sap()
    w = W.tiny()
    t = tensors("tiny")
    say("case tiny_packed_512: one call, Q = KV = 512 tokens, D=64")
    o, lse, rows, info = _run_single(sap, w.cu, w.q_segs, w.steps[0].kv_segs, t.q, t.k, t.v, 2, 2, 64, w.scale)
    assert info["n_tiles"] == 11 and len(rows) == 512
    g = np.arange(512)
    ro, rl = A.forward(f64(t.q), f64(t.k), f64(t.v), g, g, w.cu, w.scale)
    compare(o, lse, ro, rl, label="tiny")
    # the workload's inputs are fp32; the kernels take them rounded to bf16.
    # Against the oracle on the unrounded fp32 inputs the error is gated by
    # the tolerance plus what the rounding itself can move the result:
    # bf16 rounding (RNE) changes each q, k, v element by a factor 1 + a with
    # |a| <= u = 2^-9, so each logit scale q.k by at most
    #     eps_r = scale (2u + u^2) max_c sum_d |q_rd| |k_cd|    (allowed c)
    # and then every softmax weight by a factor in [e^-2eps, e^2eps]:
    #     |dO_r| <= max|v| (u + e^(2 eps_r) - 1),  |dLSE_r| <= eps_r.
    q32, k32, v32 = W.fp32_inputs_tiny()
    fo, fl = A.forward(q32, k32, v32, g, g, w.cu, w.scale)
    u = 2.0 ** -9
    allow = A.allowed(w.cu, g, g)
    q64, k64, v64 = (np.asarray(x, dtype=np.float64) for x in (q32, k32, v32))
    for h in range(2):
        eps = w.scale * (2 * u + u * u) * np.where(allow, np.abs(q64[:, h]) @ np.abs(k64[:, h]).T, 0.0).max(axis=1)
        vmax = np.array([np.abs(v64[allow[r], h]).max() for r in range(512)])
        bound_o = vmax * (u + np.expm1(2 * eps))
        err_o = np.abs(o[:, h] - fo[:, h]).max(axis=1)
        err_l = np.abs(lse[h] - fl[h])
        say(f"  tiny head {h} vs fp32-input oracle: max|dO|={err_o.max():.3e} (gate {TOL_O:.0e} + rounding bound, "
            f"worst use {(err_o / (TOL_O + bound_o)).max():.2f}), max|dLSE|={err_l.max():.3e} "
            f"(worst use {(err_l / (TOL_LSE + eps)).max():.2f})")
        assert (err_o <= TOL_O + bound_o).all() and (err_l <= TOL_LSE + eps).all()


@pytest.mark.parametrize("block_m", [128, 256])
@pytest.mark.parametrize("seed", range(10))
def test_random_small_layouts(seed, block_m):
    """Ragged tiles, 1-token and empty documents, GQA, D in {64, 128},
    non-contiguous segments, strided Q rows (and, on odd seeds, strided K / V
    rows), 128- and 256-row Q tiles; untouched rows stay NaN."""
    sap = _sap()
    rng = np.random.default_rng(900 + seed)
    d = 128 if seed % 2 else 64
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 3]))
    total = int(rng.integers(300, 1400))
    lengths = W.random_docs(rng, total, int(rng.integers(2, 500)))
    cu = W.cu_seqlens(lengths)
    a, b = sorted(rng.integers(0, total, size=2).tolist())
    b = max(b, a + 1)
    q_segs = [(a, b, 3), (0, min(a, 150), b - a + 10)] if a > 0 else [(a, b, 0)]
    q_segs = [s for s in q_segs if s[1] > s[0]]
    c0 = int(rng.integers(0, total))
    kv_segs = [(c0, total, 0), (0, c0, total - c0 + 7)] if c0 > 0 else [(0, total, 0)]
    say(f"case random seed={seed} block_m={block_m} total={total} docs={len(lengths)} hq={hq} hkv={hkv} d={d} "
        f"q={q_segs} kv={kv_segs}")
    gq = _globals(q_segs, max(ls + ge - gs for gs, ge, ls in q_segs))
    gk = _globals(kv_segs, max(ls + ge - gs for gs, ge, ls in kv_segs))
    rs = np.random.default_rng(seed)
    qf = W.bf16_round(rs.standard_normal((total, hq, d), dtype=np.float32))
    kf = W.bf16_round(rs.standard_normal((total, hkv, d), dtype=np.float32))
    vf = W.bf16_round(rs.standard_normal((total, hkv, d), dtype=np.float32))
    # local buffers; Q gets an extra padding head so its row stride exceeds hq*d
    ql = np.zeros((len(gq), hq + 1, d), dtype=np.uint16)
    ql[gq >= 0, :hq] = qf[gq[gq >= 0]]
    # K / V rows padded by an extra head on odd seeds (kv_row_stride > hkv * d)
    kpad = hkv + (seed % 2)
    kl = np.zeros((len(gk), kpad, d), dtype=np.uint16)
    vl = np.zeros((len(gk), kpad, d), dtype=np.uint16)
    kl[gk >= 0, :hkv], vl[gk >= 0, :hkv] = kf[gk[gk >= 0]], vf[gk[gk >= 0]]
    import torch
    plan = sap.sap_plan(cu, q_segs, kv_segs, block_m, 64)
    info = sap.sap_plan_info(plan)
    qd, kd, vd = to_dev(ql), to_dev(kl), to_dev(vl)
    o = torch.full((info["tq"], hq, d), float("nan"), device="cuda")
    lse = torch.full((hq, info["tq"]), float("nan"), device="cuda")
    if info["n_tiles"]:
        sap.sap_plan_upload(plan)
    sap.sap_attn_fwd(plan, qd, kd, vd, qd.stride(0), kd.stride(0), hq, hkv, d, 1.0 / np.sqrt(d), o, lse)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    touched, desc = sap.sap_plan_q_tiles(plan)
    rows = np.array([r for t in touched for r in range(desc[t, 0], desc[t, 0] + desc[t, 1])], dtype=np.int64)
    valid = np.nonzero(gq >= 0)[0]
    untouched = np.setdiff1d(np.arange(info["tq"]), rows)
    assert np.isnan(o[untouched]).all() and np.isnan(lse[:, untouched]).all(), "wrote outside touched tiles"
    q64 = np.zeros((len(gq), hq, d))
    q64[valid] = f64(qf[gq[valid]])
    ro, rl = A.forward(q64, f64(kl[:, :hkv]), f64(vl[:, :hkv]), np.where(gq >= 0, gq, 0), np.where(gk >= 0, gk, -10**9), cu,
                       1.0 / np.sqrt(d), rows=rows)
    compare(o, lse, ro, rl, rows=rows, label=f"random{seed}/{block_m}")


@pytest.mark.parametrize("block_m", [128, 256])
@pytest.mark.parametrize("hq,hkv,qscale", [(8, 2, 4.0), (3, 3, 4.0), (4, 1, 1.0)])
def test_long_documents_all_rows(hq, hkv, qscale, block_m):
    """Documents of thousands of tokens (long partner lists, many online
    softmax steps) and, with queries scaled by 4 (score spread ~16), frequent
    moves of the running max past the rescale threshold; every row."""
    sap = _sap()
    import torch
    lengths = [5000, 1, 2191, 1000]
    cu = W.cu_seqlens(lengths)
    total = int(cu[-1])
    d = 128
    scale = 1.0 / np.sqrt(d)
    say(f"case long documents {lengths} hq={hq} hkv={hkv} qscale={qscale} block_m={block_m}")
    rs = np.random.default_rng(77 + hq)
    qb = W.bf16_round(qscale * rs.standard_normal((total, hq, d), dtype=np.float32))
    kb = W.bf16_round(rs.standard_normal((total, hkv, d), dtype=np.float32))
    vb = W.bf16_round(rs.standard_normal((total, hkv, d), dtype=np.float32))
    segs = [(0, total, 0)]
    plan = sap.sap_plan(cu, segs, segs, block_m, 64)
    sap.sap_plan_upload(plan)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    o = torch.full((total, hq, d), float("nan"), device="cuda")
    lse = torch.full((hq, total), float("nan"), device="cuda")
    sap.sap_attn_fwd(plan, q, k, v, q.stride(0), k.stride(0), hq, hkv, d, scale, o, lse)
    torch.cuda.synchronize()
    g = np.arange(total)
    ro, rl = A.forward(f64(qb), f64(kb), f64(vb), g, g, cu, scale)
    compare(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, label=f"long docs hq={hq} x{qscale} bm={block_m}")
    sap.sap_plan_free(plan)


@pytest.mark.parametrize("hq,hkv,block_m", [(4, 2, 128), (4, 2, 256), (2, 1, 256), (3, 3, 128)])
def test_partner_counts_one_to_nineteen(hq, hkv, block_m):
    """One 1216-token document and Q row ranges chosen so that the Q tiles
    meet every number of 64-key partner tiles from 1 to 19, odd and even:
    the eight-wave software pipeline (its two-iteration unrolled loop and
    both of its tails) and the four-wave loop run every count."""
    sap = _sap()
    import torch
    total, d = 1216, 128
    cu = [0, total]
    rs = np.random.default_rng(77)
    qf = W.bf16_round(rs.standard_normal((total, hq, d), dtype=np.float32))
    kf = W.bf16_round(rs.standard_normal((total, hkv, d), dtype=np.float32))
    vf = W.bf16_round(rs.standard_normal((total, hkv, d), dtype=np.float32))
    counts = set()
    for a, b in [(0, 64), (0, 128), (0, 192), (0, total), (64, total), (128, total), (192, total)]:
        say(f"case partner counts hq={hq} hkv={hkv} block_m={block_m} q_rows=[{a},{b})")
        plan = sap.sap_plan(cu, [(a, b, 0)], [(0, total, 0)], block_m, 64)
        info = sap.sap_plan_info(plan)
        qt, _, _ = sap.sap_plan_tiles(plan)
        counts |= set(np.bincount(qt).tolist())
        qd, kd, vd = to_dev(qf[a:b]), to_dev(kf), to_dev(vf)
        o = torch.full((info["tq"], hq, d), float("nan"), device="cuda")
        lse = torch.full((hq, info["tq"]), float("nan"), device="cuda")
        sap.sap_plan_upload(plan)
        sap.sap_attn_fwd(plan, qd, kd, vd, qd.stride(0), kd.stride(0), hq, hkv, d, 1.0 / np.sqrt(d), o, lse)
        torch.cuda.synchronize()
        ro, rl = A.forward(f64(qf[a:b]), f64(kf), f64(vf), np.arange(a, b), np.arange(total), np.array(cu),
                           1.0 / np.sqrt(d))
        compare(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, label=f"counts/{hq}/{hkv}/{block_m}/{a}")
        sap.sap_plan_free(plan)
    assert counts == set(range(1, 20)), sorted(counts)


def test_forward_is_deterministic():
    sap = _sap()
    w = W.ring_rank(3)
    t = tensors("ring")
    q_loc = W.local_rows(t.q, w.q_segs)
    say("case ring rank3 step0 twice (bitwise)")
    a = _run_single(sap, w.cu, w.q_segs, w.steps[0].kv_segs, q_loc, t.k, t.v, 32, 32, 128, w.scale)
    b = _run_single(sap, w.cu, w.q_segs, w.steps[0].kv_segs, q_loc, t.k, t.v, 32, 32, 128, w.scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _rank_run(name, fused_merge=True):
    import torch
    from long_context_sequence_doc_amd.rank import RankForward
    w = W.by_name(name)
    t = tensors(name)
    rf = RankForward(w.cu, w.q_segs, [s.kv_segs for s in w.steps], w.hq, w.hkv, w.d, w.scale,
                     fused_merge=fused_merge)
    q = to_dev(W.local_rows(t.q, w.q_segs))
    k, v = to_dev(t.k), to_dev(t.v)
    rf.run(q, k, v, q.stride(0), k.stride(0))
    torch.cuda.synchronize()
    return w, t, rf, q, k, v


def test_ring_rank_all_steps_and_merge():
    """32K ring, rank 3: step-by-step partials and the merged result, all rows."""
    sap = _sap()
    import torch
    say("case ring_sp8_32k_rank3: 8 ring steps (2 non-empty) + merge pass")
    w, t, rf, q, k, v = _rank_run("ring", fused_merge=False)
    assert rf.active == [0, 1]
    o, lse = rf.o.cpu().numpy(), rf.lse.cpu().numpy()
    gq = w.q_global_rows()
    ro, rl = A.forward(f64(W.local_rows(t.q, w.q_segs)), f64(t.k), f64(t.v), gq, np.arange(w.total), w.cu, w.scale)
    compare(o, lse, ro, rl, label="ring merged")
    # the non-empty remote step alone
    s1 = w.steps[1]
    gk = np.concatenate([np.arange(a, b) for a, b, _ in s1.kv_segs])
    po, pl = A.forward(f64(W.local_rows(t.q, w.q_segs)), f64(t.k[gk]), f64(t.v[gk]), gq, gk, w.cu, w.scale)
    rows = np.array(rf.touched_rows(1))
    compare(rf.o_part.cpu().numpy(), rf.lse_part.cpu().numpy(), po, pl, rows=rows, label="ring step1 partial")
    rf.close()


def test_ring_rank_fused_merge():
    """32K ring, rank 3, the merge folded into the forward epilogue: all rows,
    and bit-for-bit the same rows untouched by step 1 as after step 0."""
    _sap()
    import torch
    say("case ring_sp8_32k_rank3: fused merge")
    w, t, rf, q, k, v = _rank_run("ring", fused_merge=True)
    assert rf.active == [0, 1] and rf.o_part is None
    gq = w.q_global_rows()
    ro, rl = A.forward(f64(W.local_rows(t.q, w.q_segs)), f64(t.k), f64(t.v), gq, np.arange(w.total), w.cu, w.scale)
    compare(rf.o.cpu().numpy(), rf.lse.cpu().numpy(), ro, rl, label="ring fused merge")
    rf.close()


def test_ring_rank_single_call():
    """32K ring, rank 3, every step's KV in one plan and one call (no merge):
    all rows against the oracle."""
    _sap()
    import torch
    from long_context_sequence_doc_amd.rank import RankForward
    say("case ring_sp8_32k_rank3: one call over all steps' KV")
    w = W.by_name("ring")
    t = tensors("ring")
    rc = RankForward.concatenated(w.cu, w.q_segs, [s.kv_segs for s in w.steps], w.hq, w.hkv, w.d, w.scale)
    q = to_dev(W.local_rows(t.q, w.q_segs))
    k, v = to_dev(t.k), to_dev(t.v)
    rc.run(q, k, v, q.stride(0), k.stride(0))
    torch.cuda.synchronize()
    gq = w.q_global_rows()
    ro, rl = A.forward(f64(W.local_rows(t.q, w.q_segs)), f64(t.k), f64(t.v), gq, np.arange(w.total), w.cu, w.scale)
    compare(rc.o.cpu().numpy(), rc.lse.cpu().numpy(), ro, rl, label="ring single call")
    rc.close()


@pytest.mark.parametrize("block_m", [128, 256])
@pytest.mark.parametrize("seed", range(4))
def test_fused_merge_random(seed, block_m):
    """sap_attn_fwd over KV part A, then sap_attn_fwd_merge over part B, against
    the oracle over A and B together. Rows of touched tiles with no key in B
    keep their values exactly; rows with no key in A (LSE -inf) take B's."""
    sap = _sap()
    import torch
    rng = np.random.default_rng(100 + seed)
    lengths = W.random_docs(rng, int(rng.integers(200, 900)), 300)
    cu = W.cu_seqlens(lengths)
    total = int(cu[-1])
    hq, hkv, d = [(4, 2, 64), (2, 2, 128), (6, 3, 64), (4, 1, 128)][seed]
    scale = 1.0 / np.sqrt(d)
    rs = np.random.default_rng(200 + seed)
    qb = W.bf16_round(rs.standard_normal((total, hq, d), dtype=np.float32))
    kb = W.bf16_round(rs.standard_normal((total, hkv, d), dtype=np.float32))
    vb = W.bf16_round(rs.standard_normal((total, hkv, d), dtype=np.float32))
    cut = int(rng.integers(1, total))
    segs_a, segs_b = [(0, cut, 0)], [(cut, total, cut)]
    if seed % 2:
        segs_a, segs_b = segs_b, segs_a
    q_segs = [(0, total, 0)]
    say(f"case fused merge seed {seed} block_m {block_m}: T={total} docs={len(lengths)} cut={cut} hq={hq} "
        f"hkv={hkv} d={d}")
    pa = sap.sap_plan(cu, q_segs, segs_a, block_m, 64)
    pb = sap.sap_plan(cu, q_segs, segs_b, block_m, 64)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    o = torch.zeros((total, hq, d), device="cuda")
    lse = torch.full((hq, total), float("-inf"), device="cuda")
    for p in (pa, pb):
        if sap.sap_plan_info(p)["n_tiles"]:
            sap.sap_plan_upload(p)
    sap.sap_attn_fwd(pa, q, k, v, q.stride(0), k.stride(0), hq, hkv, d, scale, o, lse)
    torch.cuda.synchronize()
    o_a, l_a = o.cpu().numpy().copy(), lse.cpu().numpy().copy()
    sap.sap_attn_fwd_merge(pb, q, k, v, q.stride(0), k.stride(0), hq, hkv, d, scale, o, lse)
    torch.cuda.synchronize()
    g = np.arange(total)
    ro, rl = A.forward(f64(qb), f64(kb), f64(vb), g, g, cu, scale)
    compare(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, label=f"fused merge seed {seed}/{block_m}")
    # rows with no key in B: unchanged, bit for bit
    gb = np.concatenate([np.arange(a, b) for a, b, _ in segs_b])
    _, rl_b = A.forward(f64(qb), f64(kb[gb]), f64(vb[gb]), g, gb, cu, scale)
    keep = np.isneginf(rl_b)
    assert np.array_equal(o.cpu().numpy().transpose(1, 0, 2)[keep], o_a.transpose(1, 0, 2)[keep])
    assert np.array_equal(lse.cpu().numpy()[keep], l_a[keep])
    sap.sap_plan_free(pa)
    sap.sap_plan_free(pb)


def test_zigzag_gqa_headline_all_rows():
    """128K zigzag GQA shard (rank 3), the benchmarked configuration (merges
    folded into the forward): every row and head against the oracle."""
    _sap()
    say("case zigzag_sp8_128k_gqa_rank3: 3 non-empty steps, fused merges, every row")
    w, t, rf, q, k, v = _rank_run("zigzag")
    assert rf.active == [0, 1, 7]
    o, lse = rf.o.cpu().numpy(), rf.lse.cpu().numpy()
    rf.close()
    ro, rl, _, _, _ = full_reference("zigzag")
    compare(o, lse, ro, rl, label="zigzag merged (all rows)")


def test_zigzag_single_call_all_rows():
    """128K zigzag GQA shard (rank 3) as one launch over all non-empty steps'
    KV (concatenated plan, no merges): every row and head."""
    _sap()
    import torch
    from long_context_sequence_doc_amd.rank import RankForward
    say("case zigzag_sp8_128k_gqa_rank3: one call over all steps' KV, every row")
    w = W.by_name("zigzag")
    t = tensors("zigzag")
    rc = RankForward.concatenated(w.cu, w.q_segs, [s.kv_segs for s in w.steps], w.hq, w.hkv, w.d, w.scale)
    assert rc.active == [0]
    q = to_dev(W.local_rows(t.q, w.q_segs))
    k, v = to_dev(t.k), to_dev(t.v)
    rc.run(q, k, v, q.stride(0), k.stride(0))
    torch.cuda.synchronize()
    o, lse = rc.o.cpu().numpy(), rc.lse.cpu().numpy()
    rc.close()
    ro, rl, _, _, _ = full_reference("zigzag")
    compare(o, lse, ro, rl, label="zigzag single call (all rows)")


def test_balanced_rank_all_rows():
    """128K sequence, document-aware balanced layout (1024-row chunks from
    sap_balance, equal to the oracle's assignment), rank 3: ring steps with
    fused merges over the rank's scattered Q chunks; every row and head."""
    sap = _sap()
    import torch
    from long_context_sequence_doc_amd.rank import RankForward
    from oracle import balance as B
    z = W.zigzag_rank(3)
    owner, _ = sap.sap_balance(z.cu, 8, 1024)
    assert owner.tolist() == B.balance(z.cu, 8, 1024)[0]
    w = W.owner_rank(z, owner.tolist(), 3, 1024, "balanced")
    say(f"case balanced_sp8_128k_gqa_rank3: {len(w.q_segs)} Q segments, fused merges, every row")
    t = tensors("zigzag")
    rf = RankForward(w.cu, w.q_segs, [s.kv_segs for s in w.steps], w.hq, w.hkv, w.d, w.scale)
    q = to_dev(W.local_rows(t.q, w.q_segs))
    k, v = to_dev(t.k), to_dev(t.v)
    rf.run(q, k, v, q.stride(0), k.stride(0))
    torch.cuda.synchronize()
    o, lse = rf.o.cpu().numpy(), rf.lse.cpu().numpy()
    rf.close()
    ro, rl, _, _, _ = full_reference("balanced")
    compare(o, lse, ro, rl, label="balanced merged (all rows)")


def test_zigzag_local_then_remote_all_rows():
    """128K zigzag GQA rank 3 as two calls: its own chunks, then every remote
    chunk together with the merge in the epilogue; every row and head."""
    _sap()
    import torch
    from long_context_sequence_doc_amd.rank import RankForward
    w = W.zigzag_rank(3)
    t = tensors("zigzag")
    say("case zigzag_sp8_128k_gqa_rank3: local step + one merged call over all remote chunks, every row")
    rf = RankForward.local_then_remote(w.cu, w.q_segs, [s.kv_segs for s in w.steps], w.hq, w.hkv, w.d, w.scale)
    assert rf.active == [0, 1]
    q = to_dev(W.local_rows(t.q, w.q_segs))
    k, v = to_dev(t.k), to_dev(t.v)
    rf.run(q, k, v, q.stride(0), k.stride(0))
    torch.cuda.synchronize()
    o, lse = rf.o.cpu().numpy(), rf.lse.cpu().numpy()
    rf.close()
    ro, rl, _, _, _ = full_reference("zigzag")
    compare(o, lse, ro, rl, label="zigzag local + remote (all rows)")


def test_training_forward_all_rows():
    _sap()
    say("case train_64k_5heads forward, every row")
    w, t, rf, q, k, v = _rank_run("train")
    o, lse = rf.o.cpu().numpy(), rf.lse.cpu().numpy()
    rf.close()
    ro, rl, _, _, _ = full_reference("train")
    compare(o, lse, ro, rl, label="train fwd (all rows)")


@pytest.mark.parametrize("name", ["ulysses", "ulysses_gqa"])
def test_ulysses_sampled(name):
    """512K Ulysses head shard (4 heads, or 4 query heads sharing one KV head),
    all heads: every row of the 123 short documents, and the last 256 rows
    plus 4096 seeded rows (seed 5) of each of the two long documents."""
    _sap()
    say(f"case {W.by_name(name).name} forward, sampled rows (all short documents, long-document tails + 4096 each)")
    w, t, rf, q, k, v = _rank_run(name)
    g = np.arange(w.total)
    rows = ulysses_rows(w.cu)
    assert len(rows) > 130000
    o = rf.o.cpu().numpy()[rows]
    lse = rf.lse.cpu().numpy()[:, rows]
    rf.close()
    ro, rl = oracle_forward_rows(t.q, t.k, t.v, g, g, w.cu, w.scale, rows, label=w.name)
    compare(o, lse, ro, rl, label=w.name)


@pytest.mark.parametrize("d", [64, 128])
def test_merges_drop_neg_inf_side_with_nan(d):
    """A side whose LSE is -inf holds no keys: its O must not reach the result
    even when it holds NaN. sap_lse_merge with NaN in the O rows of -inf
    sides; sap_attn_fwd_merge into a running O of NaN with LSE -inf (every
    touched row then takes the call's own result; untouched rows stay as
    they were)."""
    sap = _sap()
    import torch
    rng = np.random.default_rng(8)
    tq, hq = 200, 2
    oa = rng.standard_normal((tq, hq, d)).astype(np.float32)
    ob = rng.standard_normal((tq, hq, d)).astype(np.float32)
    la = (2 * rng.standard_normal((hq, tq))).astype(np.float32)
    lb = (2 * rng.standard_normal((hq, tq))).astype(np.float32)
    la[0, 10:40] = -np.inf
    oa[10:40, 0] = np.nan
    lb[1, 30:70] = -np.inf
    ob[30:70, 1] = np.nan
    la[0, 100:110] = lb[0, 100:110] = -np.inf
    oa[100:110, 0] = ob[100:110, 0] = np.nan
    say(f"case merge with NaN on -inf sides, d={d}")
    t = lambda x: torch.from_numpy(x).cuda()
    da, dla = t(oa), t(la)
    sap.sap_lse_merge(None, da, dla, t(ob), t(lb), tq, hq, d)
    torch.cuda.synchronize()
    # the oracle merge of the same values with the -inf sides' O set to 0
    clean = lambda o_, l_: np.where(np.isneginf(l_).T[:, :, None], 0.0, o_)
    ro, rl = A.merge(clean(oa, la), la, clean(ob, lb), lb)
    compare(da.cpu().numpy(), dla.cpu().numpy(), ro, rl, label="merge NaN on -inf sides")
    got = da.cpu().numpy()
    assert (got[100:110, 0] == 0).all()

    say(f"case fused merge into a NaN running O with LSE -inf, d={d}")
    lengths = [300, 1, 211]
    cu = W.cu_seqlens(lengths)
    total = int(cu[-1])
    hq, hkv = 4, 2
    scale = 1.0 / np.sqrt(d)
    rs = np.random.default_rng(9)
    qb = W.bf16_round(rs.standard_normal((total, hq, d), dtype=np.float32))
    kb = W.bf16_round(rs.standard_normal((total, hkv, d), dtype=np.float32))
    vb = W.bf16_round(rs.standard_normal((total, hkv, d), dtype=np.float32))
    kv = [(100, total, 100)]
    plan = sap.sap_plan(cu, [(0, total, 0)], kv, 128, 64)
    sap.sap_plan_upload(plan)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    o = torch.full((total, hq, d), float("nan"), device="cuda")
    lse = torch.full((hq, total), float("-inf"), device="cuda")
    sap.sap_attn_fwd_merge(plan, q, k, v, q.stride(0), k.stride(0), hq, hkv, d, scale, o, lse)
    torch.cuda.synchronize()
    g = np.arange(total)
    gk = np.arange(100, total)
    ro, rl = A.forward(f64(qb), f64(kb[100:]), f64(vb[100:]), g, gk, cu, scale)
    o_h, l_h = o.cpu().numpy(), lse.cpu().numpy()
    has = np.isfinite(rl)                    # [hq, total]: rows with a key in the call
    assert np.array_equal(np.isfinite(l_h), has) and np.isneginf(l_h[~has]).all()
    rows = np.nonzero(has.all(axis=0))[0]
    compare(o_h, l_h, ro, rl, rows=rows, label="fused merge over NaN / -inf")
    # rows without a key in this call keep their running (NaN, -inf) values
    assert np.isnan(o_h.transpose(1, 0, 2)[~has]).all()
    sap.sap_plan_free(plan)


@pytest.mark.parametrize("d", [4, 32, 64, 128, 256])
def test_merge_against_oracle(d):
    """sap_lse_merge alone, every head dim it accepts: dense (plan NULL) and
    plan-restricted, with -inf rows."""
    sap = _sap()
    import torch
    rng = np.random.default_rng(3)
    tq, hq = 300, 3
    oa = rng.standard_normal((tq, hq, d)).astype(np.float32)
    ob = rng.standard_normal((tq, hq, d)).astype(np.float32)
    la = (3 * rng.standard_normal((hq, tq))).astype(np.float32)
    lb = (3 * rng.standard_normal((hq, tq))).astype(np.float32)
    la[0, :7] = -np.inf
    oa[:7, 0] = 0
    lb[1, 5:12] = -np.inf
    ob[5:12, 1] = 0
    la[2, 20:25] = -np.inf
    lb[2, 20:25] = -np.inf
    oa[20:25, 2] = 0
    ob[20:25, 2] = 0
    say(f"case merge dense 300x3x{d}")
    t = lambda x: torch.from_numpy(x).cuda()
    da, dla = t(oa), t(la)
    sap.sap_lse_merge(None, da, dla, t(ob), t(lb), tq, hq, d)
    torch.cuda.synchronize()
    ro, rl = A.merge(oa, la, ob, lb)
    compare(da.cpu().numpy(), dla.cpu().numpy(), ro, rl, label="merge dense")
    assert np.abs(da.cpu().numpy() - ro).max() < 1e-5
    # plan-restricted: rows outside touched tiles must be left as they were
    say("case merge plan-restricted")
    cu = [0, 200, 300]
    plan = sap.sap_plan(cu, [(0, 300, 0)], [(200, 300, 0)], 128, 64)   # KV = 2nd doc: touches tiles 1, 2
    sap.sap_plan_upload(plan)
    da, dla = t(oa), t(la)
    sap.sap_lse_merge(plan, da, dla, t(ob), t(lb), tq, hq, d)
    torch.cuda.synchronize()
    touched, desc = sap.sap_plan_q_tiles(plan)
    rows = np.array([r for tt in touched for r in range(desc[tt, 0], desc[tt, 0] + desc[tt, 1])])
    other = np.setdiff1d(np.arange(tq), rows)
    got = da.cpu().numpy()
    assert np.array_equal(got[other], oa[other])
    assert np.array_equal(dla.cpu().numpy()[:, other], la[:, other])
    compare(got, dla.cpu().numpy(), ro, rl, rows=rows, label="merge plan rows")

"""Pins for the oracle's backward pass (dQ, dK, dV of sum(O * dO)).

Pinned by central finite differences in fp64, by torch.autograd (float64) on
a dense formula written independently of the oracle, by closed forms for
one-token documents, by the row-sum identities of softmax gradients, and by
the ring decomposition (per-chunk calls with the final LSE sum to the full
gradient).
"""
import numpy as np
import torch

import workloads as W
from oracle import attention as A


def _inputs(rng, lengths, hq, hkv, d):
    t = sum(lengths)
    return (rng.standard_normal((t, hq, d)), rng.standard_normal((t, hkv, d)),
            rng.standard_normal((t, hkv, d)), rng.standard_normal((t, hq, d)), W.cu_seqlens(lengths))


def _full(q, k, v, do, cu, scale):
    g = np.arange(q.shape[0])
    o, lse = A.forward(q, k, v, g, g, cu, scale)
    return A.backward(q, k, v, do, o, lse, g, g, cu, scale), o, lse


def test_finite_differences(rng):
    lengths = [3, 1, 9, 5, 0, 6]
    hq, hkv, d, scale = 2, 1, 8, 0.45
    q, k, v, do, cu = _inputs(rng, lengths, hq, hkv, d)
    (dq, dk, dv), _, _ = _full(q, k, v, do, cu, scale)
    g = np.arange(q.shape[0])

    def f(qq, kk, vv):
        o, _ = A.forward(qq, kk, vv, g, g, cu, scale)
        return float((o * do).sum())

    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        idx = [tuple(rng.integers(0, s) for s in x.shape) for _ in range(20)]
        for ix in idx:
            xp, xm = x.copy(), x.copy()
            xp[ix] += h
            xm[ix] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (f(args_p["q"], args_p["k"], args_p["v"]) - f(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            assert abs(fd - grad[ix]) < 1e-7, (name, ix, fd, grad[ix])


def test_autograd_on_dense_formula(rng):
    lengths = [7, 1, 12, 4]
    hq, hkv, d, scale = 4, 2, 8, 0.3
    q, k, v, do, cu = _inputs(rng, lengths, hq, hkv, d)
    (dq, dk, dv), _, _ = _full(q, k, v, do, cu, scale)
    t = q.shape[0]
    m = torch.zeros(t, t, dtype=torch.bool)
    s0 = 0
    for L in lengths:
        m[s0:s0 + L, s0:s0 + L] = torch.ones(L, L, dtype=torch.bool).tril()
        s0 += L
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kk = tk.repeat_interleave(hq // hkv, dim=1)
    vv = tv.repeat_interleave(hq // hkv, dim=1)
    s = scale * torch.einsum("ihd,jhd->hij", tq, kk)
    s = s.masked_fill(~m, float("-inf"))
    o = torch.einsum("hij,jhd->ihd", torch.softmax(s, dim=-1), vv)
    (o * torch.tensor(do)).sum().backward()
    assert np.abs(tq.grad.numpy() - dq).max() < 1e-12
    assert np.abs(tk.grad.numpy() - dk).max() < 1e-12
    assert np.abs(tv.grad.numpy() - dv).max() < 1e-12


def test_row_sum_identities(rng):
    """Per document and KV head: sum_j dK_j = 0 and sum_j dV_j = sum_i sum_{h in g} dO_i,h."""
    lengths = [11, 30, 2, 17]
    hq, hkv, d = 4, 2, 8
    q, k, v, do, cu = _inputs(rng, lengths, hq, hkv, d)
    (dq, dk, dv), _, _ = _full(q, k, v, do, cu, 0.4)
    grp = hq // hkv
    for i in range(len(lengths)):
        s, e = cu[i], cu[i + 1]
        assert np.abs(dk[s:e].sum(axis=0)).max() < 1e-11
        for g in range(hkv):
            want = do[s:e, g * grp:(g + 1) * grp].sum(axis=(0, 1))
            assert np.abs(dv[s:e, g].sum(axis=0) - want).max() < 1e-11


def test_one_token_documents(rng):
    lengths = [1, 6, 1, 1, 4]
    q, k, v, do, cu = _inputs(rng, lengths, 2, 2, 8)
    (dq, dk, dv), _, _ = _full(q, k, v, do, cu, 0.5)
    for tok in (0, 7, 8):
        assert np.abs(dq[tok]).max() < 1e-15
        assert np.abs(dk[tok]).max() < 1e-15
        assert np.abs(dv[tok] - do[tok]).max() < 1e-15


def test_ring_steps_sum_to_full_gradient(rng):
    lengths = W.random_docs(rng, 96, 30)
    hq, hkv, d, scale = 4, 2, 8, 0.5
    q, k, v, do, cu = _inputs(rng, lengths, hq, hkv, d)
    (dq, dk, dv), o, lse = _full(q, k, v, do, cu, scale)
    t = q.shape[0]
    g = np.arange(t)
    sq, sk, sv = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    for a in range(0, t, 32):
        gk = np.arange(a, min(t, a + 32))
        pq, pk, pv = A.backward(q, k[gk], v[gk], do, o, lse, g, gk, cu, scale)
        sq += pq
        sk[gk] += pk
        sv[gk] += pv
    assert np.abs(sq - dq).max() < 1e-12
    assert np.abs(sk - dk).max() < 1e-12
    assert np.abs(sv - dv).max() < 1e-12


def test_sampled_rows_and_cols_are_exact(rng):
    """dQ rows and dK/dV rows are independent sums; the sampled form matches."""
    lengths = [40, 1, 70, 17]
    hq, hkv, d, scale = 4, 2, 8, 0.35
    q, k, v, do, cu = _inputs(rng, lengths, hq, hkv, d)
    (dq, dk, dv), o, lse = _full(q, k, v, do, cu, scale)
    g = np.arange(q.shape[0])
    rows = np.array([0, 39, 40, 41, 100, 127])
    cols = np.array([3, 40, 55, 110, 111])
    sq, sk, sv = A.backward(q, k, v, do, o, lse, g, g, cu, scale, rows=rows, cols=cols)
    assert np.abs(sq[rows] - dq[rows]).max() < 1e-13
    assert np.abs(sk[cols] - dk[cols]).max() < 1e-13
    assert np.abs(sv[cols] - dv[cols]).max() < 1e-13
    other_r = np.setdiff1d(g, rows)
    other_c = np.setdiff1d(g, cols)
    assert (sq[other_r] == 0).all() and (sk[other_c] == 0).all() and (sv[other_c] == 0).all()

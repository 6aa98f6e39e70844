"""fp64 reference for document-masked causal attention (test infrastructure only).

Notation. A call holds local query rows r (global positions gq[r]) and local
key/value rows c (global positions gk[c]) of one packed sequence whose
document boundaries are ``cu`` (cu[0] = 0, non-decreasing, cu[-1] = total).
doc(p) is the last document whose start is <= p (empty documents are thus
skipped), ds(p) = cu[doc(p)].

Mask (HSAP summary page, original abstract: packed documents must not
cross-contaminate under causal attention; AutoSP page section 2.A step 4:
masks are re-derived from global positions after sharding):

    allowed(r, c)  <=>  ds(gq[r]) <= gk[c] <= gq[r]

A token sees itself and the earlier tokens of its own document.

Forward, per query head h with KV head g = h // (Hq // Hkv) (contiguous GQA
groups; the pages never describe GQA, this is the standard grouping):

    s_c = scale * <q[r,h], k[c,g]>          over allowed c
    m = max_c s_c,  w_c = exp(s_c - m),  Z = sum_c w_c
    O[r,h] = sum_c w_c v[c,g] / Z,  LSE[h,r] = m + ln Z
    no allowed c:  O[r,h] = 0,  LSE[h,r] = -inf

Computed by document and in blocks of query rows; each block's whole score
rows are materialised and a two-pass softmax is taken (never an online one).
"""
from __future__ import annotations

import numpy as np

# Elements of one block's score matrix (rows x keys); bounds memory for long documents.
_BLOCK_ELEMS = 1 << 24
_MAX_BLOCK_ROWS = 1024


def doc_index(cu: np.ndarray, pos: np.ndarray) -> np.ndarray:
    return np.searchsorted(np.asarray(cu, dtype=np.int64), np.asarray(pos, dtype=np.int64),
                           side="right") - 1


def doc_start(cu: np.ndarray, pos: np.ndarray) -> np.ndarray:
    cu = np.asarray(cu, dtype=np.int64)
    return cu[doc_index(cu, pos)]


def allowed(cu, gq, gk) -> np.ndarray:
    """Dense mask [len(gq), len(gk)]: ds(gq[r]) <= gk[c] <= gq[r]."""
    gq = np.asarray(gq, dtype=np.int64)
    gk = np.asarray(gk, dtype=np.int64)
    ds = doc_start(cu, gq)
    return (gk[None, :] >= ds[:, None]) & (gk[None, :] <= gq[:, None])


def _blocks(rows: np.ndarray, nkeys: int):
    step = max(1, min(_MAX_BLOCK_ROWS, _BLOCK_ELEMS // max(nkeys, 1)))
    for i in range(0, len(rows), step):
        yield rows[i:i + step]


def _doc_groups(cu, gq, gk, rows):
    """Yield (query rows of one document, candidate key columns of that document)."""
    dq = doc_index(cu, gq[rows])
    dk = doc_index(cu, gk)
    for d in np.unique(dq):
        qrows = rows[dq == d]
        kcols = np.nonzero(dk == d)[0]
        yield qrows, kcols


def forward(q, k, v, gq, gk, cu, scale, rows=None):
    """Partial (or full) attention of local Q rows against this call's KV rows.

    q [Tq,Hq,D], k/v [Tkv,Hkv,D] (any float dtype; computed in fp64).
    gq [Tq], gk [Tkv]: global positions. ``rows``: optional subset of local Q
    rows to compute (rows are independent, so a subset is exact); others keep
    O = 0 and LSE = -inf.
    Returns O [Tq,Hq,D] float64 and LSE [Hq,Tq] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    gq = np.asarray(gq, dtype=np.int64)
    gk = np.asarray(gk, dtype=np.int64)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0
    group = hq // hkv
    o = np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -np.inf)
    rows = np.arange(tq) if rows is None else np.asarray(rows, dtype=np.int64)
    for qrows, kcols in _doc_groups(cu, gq, gk, rows):
        if len(kcols) == 0:
            continue
        for qb in _blocks(qrows, len(kcols)):
            mask = allowed(cu, gq[qb], gk[kcols])
            any_key = mask.any(axis=1)
            if not any_key.any():
                continue
            live = qb[any_key]
            mask = mask[any_key]
            for h in range(hq):
                g = h // group
                s = scale * (q[live, h, :] @ k[kcols, g, :].T)
                s = np.where(mask, s, -np.inf)
                m = s.max(axis=1)
                w = np.exp(s - m[:, None])          # masked entries: exp(-inf) = 0
                z = w.sum(axis=1)
                o[live, h, :] = (w @ v[kcols, g, :]) / z[:, None]
                lse[h, live] = m + np.log(z)
    return o, lse


def merge(o_a, lse_a, o_b, lse_b):
    """Exact combination of two partial results over disjoint KV sets.

    L = log(e^La + e^Lb);  O = e^(La-L) O_a + e^(Lb-L) O_b.
    A side with L = -inf holds no keys and contributes nothing; if both are
    -inf the row stays O = 0, LSE = -inf.
    o_* [T,H,D], lse_* [H,T]. Returns new arrays (fp64).
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    finite = np.isfinite(lse)
    safe = np.where(finite, lse, 0.0)
    wa = np.where(finite & np.isfinite(lse_a), np.exp(np.where(np.isfinite(lse_a), lse_a, 0.0) - safe), 0.0)
    wb = np.where(finite & np.isfinite(lse_b), np.exp(np.where(np.isfinite(lse_b), lse_b, 0.0) - safe), 0.0)
    # weights are [H,T]; outputs are [T,H,D]
    o = wa.T[:, :, None] * o_a + wb.T[:, :, None] * o_b
    return o, lse


def backward(q, k, v, do, o_final, lse_final, gq, gk, cu, scale, rows=None, cols=None):
    """Gradients of this call's share of sum(O * dO) (recompute form).

    O_final / LSE_final are the merged results over *all* KV rows of the
    sequence; this call sees only its own KV rows, so summing the calls of a
    ring gives the full gradient:

        P_rc  = exp(s_rc - LSE_final[r])  on allowed, else 0
        dV[c,g] += sum_{h in g} sum_r P_rc dO[r,h]
        dP_rc = <dO[r,h], v[c,g]>
        D_r   = <dO[r,h], O_final[r,h]>     (= sum over all keys of P dP)
        dS_rc = P_rc (dP_rc - D_r)
        dQ[r,h] += scale sum_c dS_rc k[c,g]
        dK[c,g] += scale sum_{h in g} sum_r dS_rc q[r,h]

    ``rows`` / ``cols``: optional subsets of local Q rows / KV rows. Every
    dQ row is a sum over keys and every dK/dV row a sum over queries, each
    independent of the others, so with a subset the oracle computes dQ for
    ``rows`` only (against all keys) and dK/dV for ``cols`` only (against all
    queries); the rest stay 0. Without subsets it is one pass over all pairs.

    Returns dq [Tq,Hq,D], dk [Tkv,Hkv,D], dv [Tkv,Hkv,D] (fp64).
    """
    if rows is not None or cols is not None:
        all_r = np.arange(np.asarray(q).shape[0])
        all_c = np.arange(np.asarray(k).shape[0])
        r_sel = all_r if rows is None else np.asarray(rows, dtype=np.int64)
        c_sel = all_c if cols is None else np.asarray(cols, dtype=np.int64)
        dq, _, _ = _backward_pairs(q, k, v, do, o_final, lse_final, gq, gk, cu, scale, r_sel, all_c)
        _, dk, dv = _backward_pairs(q, k, v, do, o_final, lse_final, gq, gk, cu, scale, all_r, c_sel)
        return dq, dk, dv
    return _backward_pairs(q, k, v, do, o_final, lse_final, gq, gk, cu, scale, None, None)


def _backward_pairs(q, k, v, do, o_final, lse_final, gq, gk, cu, scale, rows, cols):
    """The backward sums of ``backward`` over query rows ``rows`` x key rows
    ``cols`` (None = all)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    o_final = np.asarray(o_final, dtype=np.float64)
    lse_final = np.asarray(lse_final, dtype=np.float64)
    gq = np.asarray(gq, dtype=np.int64)
    gk = np.asarray(gk, dtype=np.int64)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.einsum("thd,thd->ht", do, o_final)
    rows = np.arange(tq) if rows is None else rows
    for qrows, kcols in _doc_groups(cu, gq, gk, rows):
        if cols is not None:
            kcols = np.intersect1d(kcols, cols)
        if len(kcols) == 0:
            continue
        for qb in _blocks(qrows, len(kcols)):
            mask = allowed(cu, gq[qb], gk[kcols])
            if not mask.any():
                continue
            for h in range(hq):
                g = h // group
                lse_r = lse_final[h, qb]
                s = scale * (q[qb, h, :] @ k[kcols, g, :].T)
                ok = mask & np.isfinite(lse_r)[:, None]
                p = np.where(ok, np.exp(np.where(ok, s - np.where(np.isfinite(lse_r), lse_r, 0.0)[:, None], 0.0)), 0.0)
                dv[kcols, g, :] += p.T @ do[qb, h, :]
                dp = do[qb, h, :] @ v[kcols, g, :].T
                ds = p * (dp - delta[h, qb][:, None])
                dq[qb, h, :] += scale * (ds @ k[kcols, g, :])
                dk[kcols, g, :] += scale * (ds.T @ q[qb, h, :])
    return dq, dk, dv

"""Pins for the oracle's forward pass (document-masked causal attention, fp64).

Each test fixes the oracle against something other than itself: a dense
brute force written from the block-diagonal causal mask, torch's
scaled_dot_product_attention (float64, CPU) on each document alone, closed
forms, and invariants that follow from the definition (softmax rows sum to
one, shift invariance, no contamination across documents or from the future).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import workloads as W
from oracle import attention as A


def _tiny_inputs():
    w = W.tiny()
    t = W.make_tensors(w)
    f = lambda b: W.bf16_to_f32(b).astype(np.float64)
    return w, f(t.q), f(t.k), f(t.v)


def _dense_mask_from_lengths(lengths):
    """Block-diagonal lower-triangular mask built document by document."""
    n = sum(lengths)
    m = np.zeros((n, n), dtype=bool)
    s = 0
    for L in lengths:
        m[s:s + L, s:s + L] = np.tril(np.ones((L, L), dtype=bool))
        s += L
    return m


def _brute(q, k, v, lengths, scale):
    """Full T x T masked softmax per head with scipy; MHA only."""
    m = _dense_mask_from_lengths(lengths)
    t, h, d = q.shape
    o = np.zeros_like(q)
    lse = np.zeros((h, t))
    for hh in range(h):
        s = scale * np.einsum("id,jd->ij", q[:, hh], k[:, hh])
        s = np.where(m, s, -np.inf)
        p = scipy.special.softmax(s, axis=1)
        o[:, hh] = p @ v[:, hh]
        lse[hh] = scipy.special.logsumexp(s, axis=1)
    return o, lse


def test_tiny_matches_dense_brute_force():
    w, q, k, v = _tiny_inputs()
    g = np.arange(w.total)
    o, lse = A.forward(q, k, v, g, g, w.cu, w.scale)
    ob, lb = _brute(q, k, v, w.lengths, w.scale)
    assert np.abs(o - ob).max() < 1e-12
    assert np.abs(lse - lb).max() < 1e-12


def test_each_document_equals_torch_sdpa_causal():
    """Textbook special case: one document alone is plain causal attention."""
    w, q, k, v = _tiny_inputs()
    g = np.arange(w.total)
    o, lse = A.forward(q, k, v, g, g, w.cu, w.scale)
    cu = w.cu
    for d in range(len(w.lengths)):
        s, e = cu[d], cu[d + 1]
        tq = torch.from_numpy(q[s:e]).permute(1, 0, 2)[None]
        tk = torch.from_numpy(k[s:e]).permute(1, 0, 2)[None]
        tv = torch.from_numpy(v[s:e]).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=w.scale)
        ref = ref[0].permute(1, 0, 2).numpy()
        assert np.abs(o[s:e] - ref).max() < 1e-12
        # LSE of the same rows from the causal scores of this document alone
        sc = w.scale * torch.einsum("hid,hjd->hij", tq[0], tk[0])
        sc = sc.masked_fill(~torch.ones(e - s, e - s, dtype=torch.bool).tril(), float("-inf"))
        ref_lse = torch.logsumexp(sc, dim=-1).numpy()
        assert np.abs(lse[:, s:e] - ref_lse).max() < 1e-12


def test_packed_equals_documents_run_alone(rng):
    lengths = [5, 1, 17, 0, 9, 33]
    t, h, d = sum(lengths), 3, 8
    q, k, v = (rng.standard_normal((t, h, d)) for _ in range(3))
    cu = W.cu_seqlens(lengths)
    g = np.arange(t)
    o, lse = A.forward(q, k, v, g, g, cu, 0.37)
    for i, L in enumerate(lengths):
        if L == 0:
            continue
        s = cu[i]
        gl = np.arange(L)
        oo, ll = A.forward(q[s:s + L], k[s:s + L], v[s:s + L], gl, gl, np.array([0, L]), 0.37)
        assert np.abs(o[s:s + L] - oo).max() < 1e-13
        assert np.abs(lse[:, s:s + L] - ll).max() < 1e-13


def test_one_token_document_closed_form(rng):
    lengths = [4, 1, 6]
    t, h, d = 11, 2, 5
    q, k, v = (rng.standard_normal((t, h, d)) for _ in range(3))
    cu = W.cu_seqlens(lengths)
    g = np.arange(t)
    o, lse = A.forward(q, k, v, g, g, cu, 0.5)
    # token 4 is a document of its own: it sees only itself
    assert np.allclose(o[4], v[4], atol=1e-15)
    assert np.allclose(lse[:, 4], 0.5 * np.einsum("hd,hd->h", q[4], k[4]), atol=1e-14)


def test_equal_keys_closed_form(rng):
    """All keys of a document equal k: uniform weights over the causal prefix."""
    lengths = [3, 7]
    t, h, d = 10, 1, 4
    q = rng.standard_normal((t, h, d))
    v = rng.standard_normal((t, h, d))
    kvec = rng.standard_normal(d)
    k = np.broadcast_to(kvec, (t, h, d)).copy()
    cu = W.cu_seqlens(lengths)
    g = np.arange(t)
    scale = 0.8
    o, lse = A.forward(q, k, v, g, g, cu, scale)
    for i in range(t):
        ds = 0 if i < 3 else 3
        assert np.allclose(o[i, 0], v[ds:i + 1, 0].mean(axis=0), atol=1e-14)
        assert abs(lse[0, i] - (scale * q[i, 0] @ kvec + math.log(i - ds + 1))) < 1e-13


def test_rows_sum_to_one(rng):
    lengths = [13, 2, 40, 1]
    t, h, d = sum(lengths), 2, 6
    q, k = (rng.standard_normal((t, h, d)) for _ in range(2))
    cu = W.cu_seqlens(lengths)
    g = np.arange(t)
    o, _ = A.forward(q, k, np.ones((t, h, d)), g, g, cu, 1.3)
    assert np.abs(o - 1.0).max() < 1e-14


def test_key_shift_invariance(rng):
    lengths = [20, 12]
    t, h, d = 32, 2, 8
    q, k, v = (rng.standard_normal((t, h, d)) for _ in range(3))
    u = rng.standard_normal((h, d))
    cu = W.cu_seqlens(lengths)
    g = np.arange(t)
    scale = 0.35
    o1, l1 = A.forward(q, k, v, g, g, cu, scale)
    o2, l2 = A.forward(q, k + u[None], v, g, g, cu, scale)
    assert np.abs(o1 - o2).max() < 1e-12
    assert np.abs(l2 - (l1 + scale * np.einsum("thd,hd->ht", q, u))).max() < 1e-12


def test_no_contamination_from_future_or_other_documents(rng):
    lengths = [10, 15, 7]
    t, h, d = 32, 2, 4
    q, k, v = (rng.standard_normal((t, h, d)) for _ in range(3))
    cu = W.cu_seqlens(lengths)
    g = np.arange(t)
    o, lse = A.forward(q, k, v, g, g, cu, 0.6)
    i = 17  # in document 1 = [10, 25)
    k2, v2 = k.copy(), v.copy()
    k2[:10] += 5.0
    v2[:10] -= 3.0          # previous document
    k2[18:] *= -2.0
    v2[18:] += 7.0          # future tokens and the next document
    o2, lse2 = A.forward(q, k2, v2, g, g, cu, 0.6)
    assert np.array_equal(o[i], o2[i]) and np.array_equal(lse[:, i], lse2[:, i])
    # while a key inside the row's own causal window does change it
    k3 = k.copy()
    k3[12] += 1.0
    o3, _ = A.forward(q, k3, v, g, g, cu, 0.6)
    assert not np.array_equal(o[i], o3[i])


def test_gqa_equals_repeated_kv_heads(rng):
    lengths = [9, 23]
    t, hq, hkv, d = 32, 6, 2, 8
    q = rng.standard_normal((t, hq, d))
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    cu = W.cu_seqlens(lengths)
    g = np.arange(t)
    o, lse = A.forward(q, k, v, g, g, cu, 0.4)
    o2, lse2 = A.forward(q, np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1), g, g, cu, 0.4)
    assert np.abs(o - o2).max() < 1e-14 and np.abs(lse - lse2).max() < 1e-14


def test_row_subset_is_exact(rng):
    lengths = [50, 30, 20]
    t, h, d = 100, 2, 8
    q, k, v = (rng.standard_normal((t, h, d)) for _ in range(3))
    cu = W.cu_seqlens(lengths)
    g = np.arange(t)
    o, lse = A.forward(q, k, v, g, g, cu, 0.5)
    rows = np.array([0, 49, 50, 77, 99])
    o2, lse2 = A.forward(q, k, v, g, g, cu, 0.5, rows=rows)
    # rows are independent; only BLAS blocking (summation order) may differ
    assert np.abs(o[rows] - o2[rows]).max() < 1e-14 and np.abs(lse[:, rows] - lse2[:, rows]).max() < 1e-14
    others = np.setdiff1d(np.arange(t), rows)
    assert (o2[others] == 0).all() and np.isneginf(lse2[:, others]).all()


def test_rows_without_keys_are_zero_and_neg_inf(rng):
    """A call whose KV rows miss a query's window leaves O = 0, LSE = -inf."""
    lengths = [64, 64]
    t, h, d = 128, 1, 4
    q, k, v = (rng.standard_normal((t, h, d)) for _ in range(3))
    cu = W.cu_seqlens(lengths)
    gq = np.arange(64, 128)          # second document's queries
    gk = np.arange(0, 64)            # first document's keys only
    o, lse = A.forward(q[64:], k[:64], v[:64], gq, gk, cu, 0.5)
    assert (o == 0).all() and np.isneginf(lse).all()


def test_sharded_rows_use_global_positions(rng):
    """A Q shard with local rows != global positions gives the same rows."""
    lengths = [40, 25, 35]
    t, h, d = 100, 2, 8
    q, k, v = (rng.standard_normal((t, h, d)) for _ in range(3))
    cu = W.cu_seqlens(lengths)
    g = np.arange(t)
    o, lse = A.forward(q, k, v, g, g, cu, 0.5)
    gq = np.concatenate([np.arange(30, 50), np.arange(80, 100)])
    o2, lse2 = A.forward(q[gq], k, v, gq, g, cu, 0.5)
    assert np.abs(o2 - o[gq]).max() < 1e-13 and np.abs(lse2 - lse[:, gq]).max() < 1e-13

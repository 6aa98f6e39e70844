"""The allocation-free backward (sap_attn_bwd_noalloc) against the workspace
form (sap_attn_bwd) and the oracle, through the C ABI: two calls in a row on
one GPU, the second on a smaller input, so the fixed scratch is reused with
the first call's contents still in it."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from tests.gpu_common import TOL_O, f64, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _case(sap, lengths, hq, hkv, d, seed):
    import torch
    cu = W.cu_seqlens(lengths)
    total = int(cu[-1])
    scale = 1.0 / np.sqrt(d)
    rs = np.random.default_rng(seed)
    mk = lambda h: W.bf16_round(rs.standard_normal((total, h, d), dtype=np.float32))
    qb, kb, vb, dob = mk(hq), mk(hkv), mk(hkv), mk(hq)
    segs = [(0, total, 0)]
    plan = sap.sap_plan(cu, segs, segs, 64, 128)
    sap.sap_plan_upload(plan)
    need = sap.sap_attn_bwd_workspace(plan, hq, hkv, d)
    assert sap.sap_attn_bwd_workspace(plan, 0, hkv, d) > 0, "the case must split KV tiles (partial-sum slots)"
    assert need <= sap.SAP_BWD_NOALLOC_MAX_BYTES
    fplan = sap.sap_plan(cu, segs, segs, 128, 64)
    sap.sap_plan_upload(fplan)
    qd, kd, vd, dod = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(dob)
    o = torch.empty((total, hq, d), device="cuda")
    lse = torch.empty((hq, total), device="cuda")
    sap.sap_attn_fwd(fplan, qd, kd, vd, qd.stride(0), kd.stride(0), hq, hkv, d, scale, o, lse)
    g = np.arange(total)
    o_ref, lse_ref = A.forward(f64(qb), f64(kb), f64(vb), g, g, cu, scale)
    ref = A.backward(f64(qb), f64(kb), f64(vb), f64(dob), o_ref, lse_ref, g, g, cu, scale)
    # the workspace form
    ws = torch.empty(need // 4 + 64, dtype=torch.float32, device="cuda")
    want = [torch.zeros((total, hq, d), device="cuda"), torch.zeros((total, hkv, d), device="cuda"),
            torch.zeros((total, hkv, d), device="cuda")]
    sap.sap_attn_bwd(plan, qd, kd, vd, o, lse, dod, qd.stride(0), kd.stride(0), hq, hkv, d, scale, *want,
                     ws, ws.numel() * 4)
    torch.cuda.synchronize()
    return dict(plan=plan, fplan=fplan, q=qd, k=kd, v=vd, do=dod, o=o, lse=lse, hq=hq, hkv=hkv, d=d, scale=scale,
                total=total, want=want, ref=ref, need=need)


def _noalloc(sap, c):
    import torch
    got = [torch.zeros((c["total"], c["hq"], c["d"]), device="cuda"),
           torch.zeros((c["total"], c["hkv"], c["d"]), device="cuda"),
           torch.zeros((c["total"], c["hkv"], c["d"]), device="cuda")]
    sap.sap_attn_bwd_noalloc(c["plan"], c["q"], c["k"], c["v"], c["o"], c["lse"], c["do"], c["q"].stride(0),
                             c["k"].stride(0), c["hq"], c["hkv"], c["d"], c["scale"], *got)
    torch.cuda.synchronize()
    return got


def _same(c, got, label):
    import torch
    for name, a, b, r in zip(("dQ", "dK", "dV"), got, c["want"], c["ref"]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{label} {name}: differs from sap_attn_bwd"
        err = float(np.abs(a.cpu().numpy().astype(np.float64) - r).max())
        say(f"  {label} {name}: bit-identical to sap_attn_bwd; max|err| vs oracle {err:.3e}")
        assert err <= TOL_O


def test_noalloc_backward_two_calls_second_smaller():
    need_gpu()
    import long_context_sequence_doc_amd as sap
    big = _case(sap, [3000, 5, 1091], 8, 2, 128, 31)
    small = _case(sap, [2100], 4, 1, 64, 32)
    say(f"case noalloc: first call needs {big['need']} B of scratch, second {small['need']} B "
        f"(limit {sap.SAP_BWD_NOALLOC_MAX_BYTES})")
    assert small["need"] < big["need"]
    _same(big, _noalloc(sap, big), "first (larger)")
    _same(small, _noalloc(sap, small), "second (smaller)")
    # and once more, the larger again after the smaller
    _same(big, _noalloc(sap, big), "third (larger again)")
    for c in (big, small):
        sap.sap_plan_free(c["plan"])
        sap.sap_plan_free(c["fplan"])


def test_noalloc_refuses_plans_beyond_its_scratch():
    need_gpu()
    import torch
    import long_context_sequence_doc_amd as sap
    # 32 query / 16 KV heads, one 8192-token document, Q = its second half
    # against KV = its first half: 128 partial-sum slots x 16 heads x 64 KiB
    plan = sap.sap_plan([0, 8192], [(4096, 8192, 0)], [(0, 4096, 0)], 64, 128)
    sap.sap_plan_upload(plan)
    assert sap.sap_attn_bwd_workspace(plan, 32, 16, 128) > sap.SAP_BWD_NOALLOC_MAX_BYTES
    sentinel = torch.full((16,), 3.0, device="cuda")
    with pytest.raises(sap.SapError) as e:
        sap.sap_attn_bwd_noalloc(plan, sentinel, sentinel, sentinel, sentinel, sentinel, sentinel, 32 * 128, 16 * 128,
                                 32, 16, 128, 0.088, sentinel, sentinel, sentinel)
    assert e.value.status == sap.SAP_ERR_UNSUPPORTED and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (sentinel == 3.0).all()
    sap.sap_plan_free(plan)

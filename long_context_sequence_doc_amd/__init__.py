"""Document-masked causal attention for one sequence-parallel rank on MI355X.

Thin ctypes binding over ``libsap.so`` (see ``include/sap.h``): the functions
below carry the C ABI's names and only marshal arguments -- every step of the
computation runs in the library's host planner and gfx950 HIP kernels. Torch
tensors are accepted for device buffers (their data pointers are passed) and
torch's current stream is used when no stream is given.

There is no fallback: if ``libsap.so`` is missing the import of this package
fails loudly; build it with ``python long_context_sequence_doc_amd/build.py``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "SapError", "Segment", "PlanStats", "Plan",
    "sap_plan", "sap_plan_upload", "sap_plan_info", "sap_plan_tiles", "sap_plan_q_tiles",
    "sap_plan_free", "sap_balance", "sap_attn_fwd", "sap_attn_fwd_merge", "sap_lse_merge", "sap_attn_bwd_workspace", "sap_attn_bwd",
    "sap_attn_bwd_rowterm", "sap_attn_bwd_accumulate", "sap_attn_bwd_dkdv", "sap_attn_bwd_dq",
    "sap_attn_bwd_noalloc", "SAP_BWD_NOALLOC_MAX_BYTES",
    "sap_last_error", "sap_version", "lib_path", "SAP_TILE_FULL", "SAP_TILE_DIAGONAL",
    "SAP_TILE_PARTIAL",
]

SAP_OK, SAP_ERR_INVALID_ARG, SAP_ERR_UNSUPPORTED, SAP_ERR_NO_MEMORY, SAP_ERR_HIP, SAP_ERR_STATE = range(6)
SAP_TILE_FULL, SAP_TILE_DIAGONAL, SAP_TILE_PARTIAL = 0, 1, 2
SAP_BWD_NOALLOC_MAX_BYTES = 64 << 20   # the fixed scratch of sap_attn_bwd_noalloc (include/sap.h)
_STATUS = {0: "SAP_OK", 1: "SAP_ERR_INVALID_ARG", 2: "SAP_ERR_UNSUPPORTED", 3: "SAP_ERR_NO_MEMORY",
           4: "SAP_ERR_HIP", 5: "SAP_ERR_STATE"}

lib_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsap.so")
if not os.path.exists(lib_path):
    raise ImportError(f"{lib_path} is not built; run `python long_context_sequence_doc_amd/build.py`")
# torch ships its own HIP runtime (same soname, libamdhip64.so.7, but loaded
# by another file name). Loading torch first makes libsap.so bind to that one
# runtime; loading libsap.so first would put two HIP runtimes in the process,
# and the second would find no device.
import torch  # noqa: E402,F401
_lib = ctypes.CDLL(lib_path)


class SapError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class Segment(ctypes.Structure):
    _fields_ = [("global_start", ctypes.c_int32), ("global_end", ctypes.c_int32),
                ("local_start", ctypes.c_int32)]


class PlanStats(ctypes.Structure):
    _fields_ = [("n_tiles", ctypes.c_int64), ("n_full", ctypes.c_int64), ("n_diagonal", ctypes.c_int64),
                ("n_partial", ctypes.c_int64), ("useful_pairs_per_head", ctypes.c_int64),
                ("n_q_tiles", ctypes.c_int32), ("n_kv_tiles", ctypes.c_int32),
                ("n_touched_q_tiles", ctypes.c_int32), ("n_touched_kv_tiles", ctypes.c_int32),
                ("tq", ctypes.c_int32), ("tkv", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("block_n", ctypes.c_int32), ("uploaded", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_P = ctypes.c_void_p
_i32, _i64, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_sigs = {
    "sap_plan": ([ctypes.POINTER(_i32), _i32, ctypes.POINTER(Segment), _i32, ctypes.POINTER(Segment), _i32,
                  _i32, _i32, ctypes.POINTER(_P)], _i32),
    "sap_plan_upload": ([_P, _P], _i32),
    "sap_plan_info": ([_P, ctypes.POINTER(PlanStats)], _i32),
    "sap_plan_tiles": ([_P, _P, _P, _P, _i64], _i32),
    "sap_plan_q_tiles": ([_P, _P, _i32, _P, _i32], _i32),
    "sap_plan_free": ([_P], None),
    "sap_balance": ([ctypes.POINTER(_i32), _i32, _i32, _i32, _P, _i64, _P], _i32),
    "sap_attn_fwd": ([_P, _P, _P, _P, _i64, _i64, _i32, _i32, _i32, _f32, _P, _P, _P], _i32),
    "sap_attn_fwd_merge": ([_P, _P, _P, _P, _i64, _i64, _i32, _i32, _i32, _f32, _P, _P, _P], _i32),
    "sap_lse_merge": ([_P, _P, _P, _P, _P, _i32, _i32, _i32, _P], _i32),
    "sap_attn_bwd_workspace": ([_P, _i32, _i32, _i32], _sz),
    "sap_attn_bwd": ([_P, _P, _P, _P, _P, _P, _P, _i64, _i64, _i32, _i32, _i32, _f32, _P, _P, _P, _P, _sz, _P],
                     _i32),
    "sap_attn_bwd_rowterm": ([_P, _P, _P, _i64, _i32, _i32, _P, _P], _i32),
    "sap_attn_bwd_accumulate": ([_P, _P, _P, _P, _P, _P, _P, _i64, _i64, _i32, _i32, _i32, _f32, _P, _P, _P, _P,
                                 _sz, _P], _i32),
    "sap_attn_bwd_dkdv": ([_P, _P, _P, _P, _P, _P, _P, _i64, _i64, _i32, _i32, _i32, _f32, _P, _P, _P, _sz, _P],
                          _i32),
    "sap_attn_bwd_dq": ([_P, _P, _P, _P, _P, _P, _P, _i64, _i64, _i32, _i32, _i32, _f32, _P, _P], _i32),
    "sap_attn_bwd_noalloc": ([_P, _P, _P, _P, _P, _P, _P, _i64, _i64, _i32, _i32, _i32, _f32, _P, _P, _P, _P],
                             _i32),
    "sap_last_error": ([], ctypes.c_char_p),
    "sap_version": ([], _i32),
}
for _name, (_args, _ret) in _sigs.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _ret

EXPORTED = tuple(_sigs)


def sap_last_error() -> str:
    return _lib.sap_last_error().decode()


def sap_version() -> int:
    return int(_lib.sap_version())


def _check(status: int):
    if status != SAP_OK:
        raise SapError(status, sap_last_error())


def _ptr(x):
    """Device pointer of a tensor (or an int address, or None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Owning handle of a ``sap_plan_t``; freed on ``free()`` or garbage collection."""

    def __init__(self, handle: int):
        self.handle = handle

    @property
    def _as_parameter_(self):
        return self.handle

    def free(self):
        if self.handle:
            _lib.sap_plan_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def _segments(segs):
    arr = (Segment * max(len(segs), 1))()
    for i, (gs, ge, ls) in enumerate(segs):
        arr[i] = Segment(int(gs), int(ge), int(ls))
    return arr, len(segs)


def sap_plan(cu_seqlens, q_segs, kv_segs, block_m: int, block_n: int) -> Plan:
    """Host plan of one call. ``cu_seqlens``: sequence of ints; segments: (gs, ge, ls) triples."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    qa, nq = _segments(q_segs)
    ka, nk = _segments(kv_segs)
    out = _P()
    _check(_lib.sap_plan(cu.ctypes.data_as(ctypes.POINTER(_i32)), len(cu) - 1, qa, nq, ka, nk,
                         block_m, block_n, ctypes.byref(out)))
    return Plan(out.value)


def sap_plan_upload(plan: Plan, stream=None):
    _check(_lib.sap_plan_upload(plan.handle, _stream(stream)))


def sap_plan_info(plan: Plan) -> dict:
    st = PlanStats()
    _check(_lib.sap_plan_info(plan.handle, ctypes.byref(st)))
    return st.as_dict()


def sap_plan_tiles(plan: Plan):
    n = sap_plan_info(plan)["n_tiles"]
    q = np.zeros(max(n, 1), dtype=np.int32)
    k = np.zeros(max(n, 1), dtype=np.int32)
    c = np.zeros(max(n, 1), dtype=np.uint8)
    _check(_lib.sap_plan_tiles(plan.handle, q.ctypes.data, k.ctypes.data, c.ctypes.data, max(n, 1)))
    return q[:n], k[:n], c[:n]


def sap_plan_q_tiles(plan: Plan):
    info = sap_plan_info(plan)
    t = np.zeros(max(info["n_touched_q_tiles"], 1), dtype=np.int32)
    d = np.zeros(max(3 * info["n_q_tiles"], 1), dtype=np.int32)
    _check(_lib.sap_plan_q_tiles(plan.handle, t.ctypes.data, len(t), d.ctypes.data, len(d)))
    return t[:info["n_touched_q_tiles"]], d[:3 * info["n_q_tiles"]].reshape(-1, 3)


def sap_plan_free(plan: Plan):
    plan.free()


def sap_balance(cu_seqlens, n_ranks: int, chunk_rows: int):
    """Owner rank of every ``chunk_rows`` chunk (int32 array) and each rank's work (int64 array)."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    total = int(cu[-1])
    n_chunks = total // chunk_rows if chunk_rows > 0 else 0
    owner = np.zeros(max(n_chunks, 1), dtype=np.int32)
    work = np.zeros(max(n_ranks, 1), dtype=np.int64)
    _check(_lib.sap_balance(cu.ctypes.data_as(ctypes.POINTER(_i32)), len(cu) - 1, n_ranks, chunk_rows,
                            owner.ctypes.data, len(owner), work.ctypes.data))
    return owner[:n_chunks], work[:n_ranks]


def sap_attn_fwd(plan: Plan, q, k, v, q_row_stride: int, kv_row_stride: int, hq: int, hkv: int, d: int,
                 scale: float, o, lse, stream=None):
    _check(_lib.sap_attn_fwd(plan.handle, _ptr(q), _ptr(k), _ptr(v), q_row_stride, kv_row_stride, hq, hkv, d,
                             scale, _ptr(o), _ptr(lse), _stream(stream)))


def sap_attn_fwd_merge(plan: Plan, q, k, v, q_row_stride: int, kv_row_stride: int, hq: int, hkv: int, d: int,
                       scale: float, o_acc, lse_acc, stream=None):
    _check(_lib.sap_attn_fwd_merge(plan.handle, _ptr(q), _ptr(k), _ptr(v), q_row_stride, kv_row_stride, hq, hkv, d,
                                   scale, _ptr(o_acc), _ptr(lse_acc), _stream(stream)))


def sap_lse_merge(plan, o_acc, lse_acc, o_part, lse_part, tq: int, hq: int, d: int, stream=None):
    _check(_lib.sap_lse_merge(plan.handle if plan is not None else None, _ptr(o_acc), _ptr(lse_acc),
                              _ptr(o_part), _ptr(lse_part), tq, hq, d, _stream(stream)))


def sap_attn_bwd_workspace(plan: Plan, hq: int, hkv: int, d: int) -> int:
    return int(_lib.sap_attn_bwd_workspace(plan.handle, hq, hkv, d))


def sap_attn_bwd(plan: Plan, q, k, v, o, lse_final, dout, q_row_stride: int, kv_row_stride: int, hq: int,
                 hkv: int, d: int, scale: float, dq, dk, dv, workspace, workspace_bytes: int, stream=None):
    _check(_lib.sap_attn_bwd(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_final), _ptr(dout),
                             q_row_stride, kv_row_stride, hq, hkv, d, scale, _ptr(dq), _ptr(dk), _ptr(dv),
                             _ptr(workspace), workspace_bytes, _stream(stream)))


def sap_attn_bwd_rowterm(plan: Plan, o, dout, q_row_stride: int, hq: int, d: int, delta, stream=None):
    _check(_lib.sap_attn_bwd_rowterm(plan.handle, _ptr(o), _ptr(dout), q_row_stride, hq, d, _ptr(delta),
                                     _stream(stream)))


def sap_attn_bwd_accumulate(plan: Plan, q, k, v, lse_final, delta, dout, q_row_stride: int, kv_row_stride: int,
                            hq: int, hkv: int, d: int, scale: float, dq, dk, dv, workspace=None,
                            workspace_bytes: int = 0, stream=None):
    _check(_lib.sap_attn_bwd_accumulate(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(lse_final), _ptr(delta),
                                        _ptr(dout), q_row_stride, kv_row_stride, hq, hkv, d, scale, _ptr(dq),
                                        _ptr(dk), _ptr(dv), _ptr(workspace), workspace_bytes, _stream(stream)))


def sap_attn_bwd_dkdv(plan: Plan, q, k, v, lse_final, delta, dout, q_row_stride: int, kv_row_stride: int, hq: int,
                      hkv: int, d: int, scale: float, dk, dv, workspace=None, workspace_bytes: int = 0, stream=None):
    _check(_lib.sap_attn_bwd_dkdv(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(lse_final), _ptr(delta), _ptr(dout),
                                  q_row_stride, kv_row_stride, hq, hkv, d, scale, _ptr(dk), _ptr(dv), _ptr(workspace),
                                  workspace_bytes, _stream(stream)))


def sap_attn_bwd_dq(plan: Plan, q, k, v, lse_final, delta, dout, q_row_stride: int, kv_row_stride: int, hq: int,
                    hkv: int, d: int, scale: float, dq, stream=None):
    _check(_lib.sap_attn_bwd_dq(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(lse_final), _ptr(delta), _ptr(dout),
                                q_row_stride, kv_row_stride, hq, hkv, d, scale, _ptr(dq), _stream(stream)))


def sap_attn_bwd_noalloc(plan: Plan, q, k, v, o, lse_final, dout, q_row_stride: int, kv_row_stride: int, hq: int,
                         hkv: int, d: int, scale: float, dq, dk, dv, stream=None):
    _check(_lib.sap_attn_bwd_noalloc(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_final), _ptr(dout),
                                     q_row_stride, kv_row_stride, hq, hkv, d, scale, _ptr(dq), _ptr(dk), _ptr(dv),
                                     _stream(stream)))

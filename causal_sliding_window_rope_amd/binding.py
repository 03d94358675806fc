"""Thin ctypes binding of libswa (the C ABI declared in include/swa.h).

Argument marshalling only: every function takes torch tensors that already live on the GPU,
checks their dtype / shape / contiguity, and passes raw device pointers plus the current HIP
stream to the library. All computation happens in the library's HIP kernels. If the library
is not built, every call raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SWA_LIB names another build of the same library (e.g. one compiled with different options)
LIB_PATH = os.environ.get("SWA_LIB") or os.path.join(_PKG, "libswa.so")

SWA_F32, SWA_BF16 = 0, 1
SWA_WINDOW_FULL = -1
STATUS = {0: "SWA_OK", 1: "SWA_ERR_INVALID_ARG", 2: "SWA_ERR_UNSUPPORTED", 3: "SWA_ERR_ALIGN",
          4: "SWA_ERR_WORKSPACE", 5: "SWA_ERR_HIP"}

# exported symbol -> (restype, argtypes); must match include/swa.h
_P, _I, _F, _D, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
SIGNATURES = {
    "swa_last_error": (ctypes.c_char_p, []),
    "swa_version": (ctypes.c_char_p, []),
    "rope_table": (_I, [_P, _I, _I, _D, _P]),
    "rope_qknorm_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "rope_qknorm_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "ve_gate_v": (_I, [_P, _I, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P]),
    "ve_gate_dv": (_I, [_P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "ve_gate_v_bwd_workspace_size": (_S, [_I, _I, _I]),
    "ve_gate_v_bwd": (_I, [_P, _I, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _P]),
    "swa_doc_bounds": (_I, [_P, _P, _I, _I, _P]),
    "swa_fwd": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "swa_bwd_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "swa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S,
                     _I, _I, _I, _I, _I, _F, _I, _P]),
    "swa_bwd_ds_workspace_size": (_S, [_I, _I, _I, _I, _I, _I]),
    "swa_bwd_ds": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S,
                        _I, _I, _I, _I, _I, _F, _I, _P]),
    "swa_bwd_dkdv_ds": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _S,
                             _I, _I, _I, _I, _I, _F, _I, _P]),
    "swa_bwd_dq_ds": (_I, [_P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _F, _I, _P]),
    "swa_fwd_qnorm": (_I, [_P, _P, _F, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                           _F, _I, _P]),
    "swa_bwd_dq_ds_qnorm": (_I, [_P, _P, _P, _P, _F, _P, _P, _S, _I, _I, _I, _I, _I, _F, _I, _P]),
    "swa_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                             _I, _I, _I, _I, _I, _F, _I, _P]),
    "swa_bwd_preprocess": (_I, [_P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _P]),
    "swa_bwd_dkdv": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _S,
                          _I, _I, _I, _I, _I, _F, _I, _P]),
    "swa_bwd_dq": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I,
                        _F, _I, _P]),
    "swa_bwd_dq_rowterms": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _S, _I, _I,
                                 _I, _I, _I, _F, _I, _P]),
    "swa_fp8_v_bytes": (_S, [_I, _I, _I, _I]),
    "rope_qknorm_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "swa_fp8_pack": (_I, [_P, _P, _P, _F, _F, _F, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "swa_fwd_fp8": (_I, [_P, _P, _P, _F, _F, _F, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "swa_decode_prologue": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "swa_decode_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "swa_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _F, _I, _P]),
}

_lib = None


class SwaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {msg}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libswa.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m causal_sliding_window_rope_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib = lib
    return lib


def _call(name: str, *args) -> int:
    lib = load()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise SwaError(name, st, lib.swa_last_error().decode())
    return st


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SWA_BF16
    if t.dtype == torch.float32:
        return SWA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(t: torch.Tensor, name: str, shape=None, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def version() -> str:
    return load().swa_version().decode()


def rope_table(T: int, D: int, base: float = 10000.0, device="cuda") -> torch.Tensor:
    cs = torch.empty((T, D // 2, 2), dtype=torch.float32, device=device)
    _call("rope_table", _ptr(cs), T, D, float(base), _stream())
    return cs


def rope_qknorm_fwd(q, k, cos_sin, eps: float = 1e-6):
    """(qn, kn); q=None processes k only and returns (None, kn)."""
    B, T, H, D = k.shape
    for t, n in ((q, "q"), (k, "k")):
        if t is not None:
            _check(t, n, (B, T, H, D), k.dtype)
    _check(cos_sin, "cos_sin", (T, D // 2, 2), torch.float32)
    qn = None if q is None else torch.empty_like(q)
    kn = torch.empty_like(k)
    _call("rope_qknorm_fwd", _ptr(q), _ptr(k), _ptr(cos_sin), _ptr(qn), _ptr(kn), B, T, H, D,
          float(eps), _dt(k), _stream())
    return qn, kn


def rope_qknorm_bwd(q, k, cos_sin, dqn, dkn, eps: float = 1e-6):
    """(dq, dk); q=None and dqn=None process k only and return (None, dk)."""
    B, T, H, D = k.shape
    for t, n in ((q, "q"), (k, "k"), (dqn, "dqn"), (dkn, "dkn")):
        if t is not None:
            _check(t, n, (B, T, H, D), k.dtype)
    _check(cos_sin, "cos_sin", (T, D // 2, 2), torch.float32)
    dq = None if q is None else torch.empty_like(q)
    dk = torch.empty_like(k)
    _call("rope_qknorm_bwd", _ptr(q), _ptr(k), _ptr(cos_sin), _ptr(dqn), _ptr(dkn), _ptr(dq),
          _ptr(dk), B, T, H, D, float(eps), _dt(k), _stream())
    return dq, dk


def ve_gate_v(x, Wg, v=None, ve=None, materialize: bool = False, ve_ids=None):
    """gate (B, T, H) float32; with materialize=True also v_eff = v + gate * ve (ve_ids (B, T)
    int32: ve is a (rows, H*D) table read by token id)."""
    B, T, C = x.shape
    H = Wg.shape[1]
    _check(x, "x")
    _check(Wg, "Wg", (32, H), torch.float32)
    gate = torch.empty((B, T, H), dtype=torch.float32, device=x.device)
    D = v.shape[-1] if v is not None else 64
    ids, rows = None, 0
    if materialize:
        _check(v, "v", (B, T, H, D), x.dtype)
        if ve_ids is not None:
            _check(ve_ids, "ve_ids", (B, T), torch.int32)
            _check(ve, "ve", (ve.shape[0], H * D), x.dtype)
            ids, rows = _ptr(ve_ids), ve.shape[0]
        else:
            _check(ve, "ve", (B, T, H * D), x.dtype)
    v_eff = torch.empty_like(v) if materialize else None
    _call("ve_gate_v", _ptr(x), C, _ptr(Wg), _ptr(gate), _ptr(v if materialize else None),
          _ptr(ve if materialize else None), ids, rows, _ptr(v_eff), B, T, H, D, _dt(x),
          _stream())
    return (gate, v_eff) if materialize else gate


def ve_gate_dv(dv_eff, ve, gate, ve_ids=None, dve=None):
    """(dve, dgate) from dv_eff. Per-token mode: dve (B, T, H*D) in dv_eff's dtype. Table mode
    (ve_ids): dve is the (rows, H*D) float table gradient, accumulated into (zeroed if new)."""
    B, T, H, D = dv_eff.shape
    _check(dv_eff, "dv_eff")
    _check(gate, "gate", (B, T, H), torch.float32)
    ids, rows = None, 0
    if ve_ids is not None:
        _check(ve_ids, "ve_ids", (B, T), torch.int32)
        _check(ve, "ve", (ve.shape[0], H * D), dv_eff.dtype)
        ids, rows = _ptr(ve_ids), ve.shape[0]
        if dve is None:
            dve = torch.zeros((rows, H * D), dtype=torch.float32, device=dv_eff.device)
        _check(dve, "dve", (rows, H * D), torch.float32)
    else:
        _check(ve, "ve", (B, T, H * D), dv_eff.dtype)
        if dve is None:
            dve = torch.empty((B, T, H * D), dtype=dv_eff.dtype, device=dv_eff.device)
        _check(dve, "dve", (B, T, H * D), dv_eff.dtype)
    dgate = torch.empty((B, T, H), dtype=torch.float32, device=dv_eff.device)
    _call("ve_gate_dv", _ptr(dv_eff), _ptr(ve), ids, rows, _ptr(gate), _ptr(dve), _ptr(dgate),
          B, T, H, D, _dt(dv_eff), _stream())
    return dve, dgate


def ve_gate_v_bwd(x, Wg, gate, dgate, want_dx32: bool = True):
    B, T, C = x.shape
    H = Wg.shape[1]
    _check(x, "x")
    _check(gate, "gate", (B, T, H), torch.float32)
    _check(dgate, "dgate", (B, T, H), torch.float32)
    dWg = torch.empty((32, H), dtype=torch.float32, device=x.device)
    dx32 = torch.empty((B, T, 32), dtype=x.dtype, device=x.device) if want_dx32 else None
    nws = load().ve_gate_v_bwd_workspace_size(B, T, H)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=x.device)
    _call("ve_gate_v_bwd", _ptr(x), C, _ptr(Wg), _ptr(gate), _ptr(dgate), _ptr(dWg), _ptr(dx32),
          _ptr(ws), nws, B, T, H, _dt(x), _stream())
    return dWg, dx32


def swa_doc_bounds(doc_id, out=None):
    """Per-token [start, end) of each token's document (maximal run of equal ids), (B, T, 2)."""
    B, T = doc_id.shape
    _check(doc_id, "doc_id", (B, T), torch.int32)
    bounds = torch.empty((B, T, 2), dtype=torch.int32, device=doc_id.device) if out is None else out
    _call("swa_doc_bounds", _ptr(doc_id), _ptr(bounds), B, T, _stream())
    return bounds


def _ve_table(ve, gate, ve_ids, B, T, H, D, dtype):
    """Checks the value-embedding arguments; returns (ids pointer, table rows)."""
    if ve is None:
        if ve_ids is not None:
            raise ValueError("ve_ids needs ve and gate")
        return None, 0
    _check(gate, "gate", (B, T, H), torch.float32)
    if ve_ids is None:
        _check(ve, "ve", (B, T, H * D), dtype)
        return None, 0
    _check(ve_ids, "ve_ids", (B, T), torch.int32)
    _check(ve, "ve", (ve.shape[0], H * D), dtype)
    return _ptr(ve_ids), ve.shape[0]


def swa_fwd(q, k, v, window: int, scale: float | None = None, ve=None, gate=None, out=None,
            lse=None, doc_bounds=None, ve_ids=None):
    """ve_ids (B, T) int32 selects the table mode: ve is then a (rows, H*D) table."""
    B, T, H, D = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, (B, T, H, D), q.dtype)
    ids, rows = _ve_table(ve, gate, ve_ids, B, T, H, D, q.dtype)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if lse is None else lse
    if doc_bounds is not None:
        _check(doc_bounds, "doc_bounds", (B, T, 2), torch.int32)
    _call("swa_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(ve), _ptr(gate), ids, rows, _ptr(doc_bounds),
          _ptr(o),
          _ptr(lse), B, T, H, D, int(window), float(scale), _dt(q), _stream())
    return o, lse


def swa_fwd_qnorm(q, cos_sin, k, v, window: int, scale: float | None = None,
                  eps: float = 1e-6, ve=None, gate=None, doc_bounds=None, ve_ids=None):
    """swa_fwd with the query prologue inside the kernel: q raw, k normalised; returns
    (qn, o, lse)."""
    B, T, H, D = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, (B, T, H, D), q.dtype)
    _check(cos_sin, "cos_sin", (T, D // 2, 2), torch.float32)
    ids, rows = _ve_table(ve, gate, ve_ids, B, T, H, D, q.dtype)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    qn, o = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    if doc_bounds is not None:
        _check(doc_bounds, "doc_bounds", (B, T, 2), torch.int32)
    _call("swa_fwd_qnorm", _ptr(q), _ptr(cos_sin), float(eps), _ptr(k), _ptr(v), _ptr(ve),
          _ptr(gate), ids, rows, _ptr(doc_bounds), _ptr(qn), _ptr(o), _ptr(lse), B, T, H, D,
          int(window), float(scale), _dt(q), _stream())
    return qn, o, lse


def swa_bwd_dq_ds_qnorm(k, q, cos_sin, workspace, window: int, scale: float | None = None,
                        eps: float = 1e-6, doc_bounds=None, out=None):
    """dq w.r.t. the raw queries q from the dS stored in `workspace` by swa_bwd_dkdv_ds."""
    B, T, H, D = k.shape
    for t, n in ((q, "q"), (k, "k")):
        _check(t, n, (B, T, H, D), k.dtype)
    _check(cos_sin, "cos_sin", (T, D // 2, 2), torch.float32)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    dq = torch.empty_like(q) if out is None else out
    if doc_bounds is not None:
        _check(doc_bounds, "doc_bounds", (B, T, 2), torch.int32)
    _call("swa_bwd_dq_ds_qnorm", _ptr(k), _ptr(doc_bounds), _ptr(q), _ptr(cos_sin), float(eps),
          _ptr(dq), _ptr(workspace), workspace.numel() * workspace.element_size(), B, T, H, D,
          int(window), float(scale), _dt(k), _stream())
    return dq


def swa_bwd_workspace_size(B: int, T: int, H: int, D: int, dtype: torch.dtype) -> int:
    return load().swa_bwd_workspace_size(B, T, H, D, SWA_BF16 if dtype == torch.bfloat16 else SWA_F32)


def _grads(q, ve, ve_ids, B, T, H):
    """Fresh gradient buffers; in the table mode dve is a zeroed float table gradient."""
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    if ve is None:
        return dq, dk, dv, None, None
    if ve_ids is None:
        dve = torch.empty_like(ve)
    else:
        dve = torch.zeros(ve.shape, dtype=torch.float32, device=q.device)
    return dq, dk, dv, dve, torch.empty((B, T, H), dtype=torch.float32, device=q.device)


def swa_bwd(q, k, v, o, lse, dO, window: int, scale: float | None = None, ve=None, gate=None,
            workspace=None, grads=None, doc_bounds=None, ve_ids=None):
    """Returns (dq, dk, dv) or, with the gate, (dq, dk, dv, dve, dgate). With ve_ids, dve is the
    (rows, H*D) float table gradient, accumulated into (a given one is not zeroed)."""
    B, T, H, D = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO")):
        _check(t, n, (B, T, H, D), q.dtype)
    _check(lse, "lse", (B, H, T), torch.float32)
    ids, rows = _ve_table(ve, gate, ve_ids, B, T, H, D, q.dtype)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    ws_bytes = swa_bwd_workspace_size(B, T, H, D, q.dtype)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    dq, dk, dv, dve, dgate = _grads(q, ve, ve_ids, B, T, H) if grads is None else grads
    if doc_bounds is not None:
        _check(doc_bounds, "doc_bounds", (B, T, 2), torch.int32)
    _call("swa_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(ve), _ptr(gate), ids, rows,
          _ptr(doc_bounds), _ptr(o),
          _ptr(lse), _ptr(dO),
          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dve), _ptr(dgate), _ptr(workspace),
          workspace.numel() * workspace.element_size(), B, T, H, D, int(window), float(scale),
          _dt(q), _stream())
    if ve is not None:
        return dq, dk, dv, dve, dgate
    return dq, dk, dv


def swa_bwd_ds_workspace_size(B: int, T: int, H: int, D: int, window: int,
                              dtype: torch.dtype) -> int:
    return load().swa_bwd_ds_workspace_size(B, T, H, D, int(window),
                                            SWA_BF16 if dtype == torch.bfloat16 else SWA_F32)


def swa_bwd_ds(q, k, v, o, lse, dO, window: int, scale: float | None = None, ve=None, gate=None,
               workspace=None, grads=None, doc_bounds=None, ve_ids=None, stages: bool = False):
    """The backward with the score gradient stored (swa_bwd_ds), or with stages=True its C-ABI
    stages (preprocess, dK/dV storing dS, dq from dS). Returns as swa_bwd."""
    B, T, H, D = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO")):
        _check(t, n, (B, T, H, D), q.dtype)
    _check(lse, "lse", (B, H, T), torch.float32)
    ids, rows = _ve_table(ve, gate, ve_ids, B, T, H, D, q.dtype)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if workspace is None:
        workspace = torch.empty(swa_bwd_ds_workspace_size(B, T, H, D, window, q.dtype),
                                dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    dq, dk, dv, dve, dgate = _grads(q, ve, ve_ids, B, T, H) if grads is None else grads
    if doc_bounds is not None:
        _check(doc_bounds, "doc_bounds", (B, T, 2), torch.int32)
    st, dt = _stream(), _dt(q)
    common = (_ptr(q), _ptr(k), _ptr(v), _ptr(ve), _ptr(gate), ids, rows, _ptr(doc_bounds))
    if not stages:
        _call("swa_bwd_ds", *common, _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv),
              _ptr(dve), _ptr(dgate), _ptr(workspace), nbytes, B, T, H, D, int(window),
              float(scale), dt, st)
    else:
        _call("swa_bwd_preprocess", _ptr(o), _ptr(dO), _ptr(lse), _ptr(workspace), nbytes, B, T,
              H, D, dt, st)
        _call("swa_bwd_dkdv_ds", *common, _ptr(lse), _ptr(dO), _ptr(dk), _ptr(dv), _ptr(dve),
              _ptr(dgate), _ptr(workspace), nbytes, B, T, H, D, int(window), float(scale), dt, st)
        _call("swa_bwd_dq_ds", _ptr(k), _ptr(doc_bounds), _ptr(dq), _ptr(workspace), nbytes, B, T,
              H, D, int(window), float(scale), dt, st)
    if ve is not None:
        return dq, dk, dv, dve, dgate
    return dq, dk, dv


def swa_bwd_noalloc(q, k, v, o, lse, dO, window: int, scale: float | None = None, ve=None,
                    gate=None, grads=None, doc_bounds=None, ve_ids=None):
    """swa_bwd on the library's static scratch instead of a workspace (same results)."""
    B, T, H, D = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO")):
        _check(t, n, (B, T, H, D), q.dtype)
    _check(lse, "lse", (B, H, T), torch.float32)
    ids, rows = _ve_table(ve, gate, ve_ids, B, T, H, D, q.dtype)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    dq, dk, dv, dve, dgate = _grads(q, ve, ve_ids, B, T, H) if grads is None else grads
    if doc_bounds is not None:
        _check(doc_bounds, "doc_bounds", (B, T, 2), torch.int32)
    _call("swa_bwd_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(ve), _ptr(gate), ids, rows,
          _ptr(doc_bounds), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dve),
          _ptr(dgate), B, T, H, D, int(window), float(scale), _dt(q), _stream())
    if ve is not None:
        return dq, dk, dv, dve, dgate
    return dq, dk, dv


def rowterm_views(workspace, B: int, T: int, H: int):
    """(ndelta, nlse2) float32 (B, H, T) views of a swa_bwd workspace: the row terms -delta and
    -lse*log2(e) as the header lays them out (each array 256-byte aligned, then 512 bytes of
    slack)."""
    n = B * H * T
    blk = ((n * 4 + 255) // 256) * 256 + 512
    f = workspace.view(torch.uint8)
    nd = f[:n * 4].view(torch.float32).view(B, H, T)
    nl = f[blk:blk + n * 4].view(torch.float32).view(B, H, T)
    return nd, nl


def swa_bwd_preprocess(o, dO, lse, workspace=None):
    """Row terms of the backward into a (new or given) workspace; returns the workspace."""
    B, T, H, D = o.shape
    _check(o, "o", (B, T, H, D))
    _check(dO, "dO", (B, T, H, D), o.dtype)
    _check(lse, "lse", (B, H, T), torch.float32)
    ws_bytes = swa_bwd_workspace_size(B, T, H, D, o.dtype)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=o.device)
    _call("swa_bwd_preprocess", _ptr(o), _ptr(dO), _ptr(lse), _ptr(workspace),
          workspace.numel() * workspace.element_size(), B, T, H, D, _dt(o), _stream())
    return workspace


def swa_bwd_stages(q, k, v, o, lse, dO, window: int, scale: float | None = None, ve=None,
                   gate=None, workspace=None, grads=None, doc_bounds=None, ve_ids=None,
                   preprocess: bool = False):
    """swa_bwd as its C-ABI stages: dQ with the row terms, then dK/dV (the one-call order), or
    with preprocess=True: preprocess, dK/dV, dQ."""
    B, T, H, D = q.shape
    ids, rows = _ve_table(ve, gate, ve_ids, B, T, H, D, q.dtype)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    ws_bytes = swa_bwd_workspace_size(B, T, H, D, q.dtype)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    dq, dk, dv, dve, dgate = _grads(q, ve, ve_ids, B, T, H) if grads is None else grads
    st = _stream()
    dt = _dt(q)
    common = (_ptr(q), _ptr(k), _ptr(v), _ptr(ve), _ptr(gate), ids, rows, _ptr(doc_bounds))
    if preprocess:
        _call("swa_bwd_preprocess", _ptr(o), _ptr(dO), _ptr(lse), _ptr(workspace), nbytes, B, T, H,
              D, dt, st)
    else:
        _call("swa_bwd_dq_rowterms", *common, _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
              _ptr(workspace), nbytes, B, T, H, D, int(window), float(scale), dt, st)
    _call("swa_bwd_dkdv", *common, _ptr(lse), _ptr(dO), _ptr(dk), _ptr(dv), _ptr(dve), _ptr(dgate),
          _ptr(workspace), nbytes, B, T, H, D, int(window), float(scale), dt, st)
    if preprocess:
        _call("swa_bwd_dq", *common, _ptr(lse), _ptr(dO), _ptr(dq), _ptr(workspace), nbytes, B, T,
              H, D, int(window), float(scale), dt, st)
    if ve is not None:
        return dq, dk, dv, dve, dgate
    return dq, dk, dv


def swa_fp8_pack(q=None, k=None, v=None, q_scale: float = 1.0, k_scale: float = 1.0,
                 v_scale: float = 1.0):
    """e4m3 codes of q / q_scale, k / k_scale (uint8, (B, T, H, D)) and the packed transposed
    V operand of v / v_scale (uint8, swa_fp8_v_bytes); None for a tensor not given."""
    ref = next(t for t in (q, k, v) if t is not None)
    B, T, H, D = ref.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t is not None:
            _check(t, n, (B, T, H, D), ref.dtype)
    q8 = torch.empty((B, T, H, D), dtype=torch.uint8, device=ref.device) if q is not None else None
    k8 = torch.empty((B, T, H, D), dtype=torch.uint8, device=ref.device) if k is not None else None
    v8t = None
    if v is not None:
        v8t = torch.empty(load().swa_fp8_v_bytes(B, T, H, D), dtype=torch.uint8, device=ref.device)
    _call("swa_fp8_pack", _ptr(q), _ptr(k), _ptr(v), float(q_scale), float(k_scale),
          float(v_scale), _ptr(q8), _ptr(k8), _ptr(v8t), B, T, H, D, _dt(ref), _stream())
    return q8, k8, v8t


def rope_qknorm_fwd_fp8(q, k, cos_sin, eps: float = 1e-6):
    """q_hat, k_hat as e4m3 codes (uint8, (B, T, H, D), scale 1)."""
    B, T, H, D = q.shape
    _check(q, "q", (B, T, H, D))
    _check(k, "k", (B, T, H, D), q.dtype)
    _check(cos_sin, "cos_sin", dtype=torch.float32)
    q8 = torch.empty((B, T, H, D), dtype=torch.uint8, device=q.device)
    k8 = torch.empty_like(q8)
    _call("rope_qknorm_fwd_fp8", _ptr(q), _ptr(k), _ptr(cos_sin), _ptr(q8), _ptr(k8), B, T, H, D,
          float(eps), _dt(q), _stream())
    return q8, k8


def swa_fwd_fp8(q8, k8, v8t, window: int, q_scale: float = 1.0, k_scale: float = 1.0,
                v_scale: float = 1.0, scale: float | None = None, doc_bounds=None, out=None,
                lse=None):
    """Forward on fp8 operands from swa_fp8_pack: O (B, T, H, D) bf16 and lse (B, H, T)."""
    B, T, H, D = q8.shape
    _check(q8, "q8", (B, T, H, D), torch.uint8)
    _check(k8, "k8", (B, T, H, D), torch.uint8)
    _check(v8t, "v8t", (load().swa_fp8_v_bytes(B, T, H, D),), torch.uint8)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=q8.device) if out is None else out
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q8.device) if lse is None else lse
    if doc_bounds is not None:
        _check(doc_bounds, "doc_bounds", (B, T, 2), torch.int32)
    _call("swa_fwd_fp8", _ptr(q8), _ptr(k8), _ptr(v8t), float(q_scale), float(k_scale),
          float(v_scale), _ptr(doc_bounds), _ptr(o), _ptr(lse), B, T, H, D, int(window),
          float(scale), _stream())
    return o, lse


def swa_decode_prologue(q, k, v, cos_sin, pos, k_cache, v_cache, eps: float = 1e-6, qn=None):
    """RoPE at pos[b] + QK-norm of one new token per sequence; stores k, v in the ring caches.
    q, k, v: (B, H, D); caches: (B, cap, H, D); pos: (B,) int32. Returns qn (B, H, D)."""
    B, H, D = q.shape
    cap = k_cache.shape[1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, (B, H, D), q.dtype)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _check(t, n, (B, cap, H, D), q.dtype)
    _check(pos, "pos", (B,), torch.int32)
    _check(cos_sin, "cos_sin", (cos_sin.shape[0], D // 2, 2), torch.float32)
    qn = torch.empty_like(q) if qn is None else qn
    _call("swa_decode_prologue", _ptr(q), _ptr(k), _ptr(v), _ptr(cos_sin), cos_sin.shape[0],
          _ptr(pos), _ptr(qn), _ptr(k_cache), _ptr(v_cache), B, H, D, cap, float(eps), _dt(q),
          _stream())
    return qn


def swa_decode_workspace_size(B: int, H: int, D: int, cap: int, window: int) -> int:
    return load().swa_decode_workspace_size(B, H, D, cap, int(window))


def swa_decode(qn, k_cache, v_cache, pos, window: int, scale: float | None = None,
               workspace=None, out=None, lse=None):
    """Attention of each sequence's new query over its cached window. Returns (o, lse)."""
    B, H, D = qn.shape
    cap = k_cache.shape[1]
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _check(t, n, (B, cap, H, D), qn.dtype)
    _check(pos, "pos", (B,), torch.int32)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if workspace is None:
        n = swa_decode_workspace_size(B, H, D, cap, window)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=qn.device)
    o = torch.empty_like(qn) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=qn.device) if lse is None else lse
    _call("swa_decode", _ptr(qn), _ptr(k_cache), _ptr(v_cache), _ptr(pos), _ptr(o), _ptr(lse),
          _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, D, cap, int(window),
          float(scale), _dt(qn), _stream())
    return o, lse

"""C-ABI checks that need no GPU: the library loads, exports every function include/swa.h
declares, and rejects bad arguments on the host before any launch (only fake, never
dereferenced pointers are passed, and each call fails validation)."""

import ctypes
import os
import re
import subprocess

import pytest

from causal_sliding_window_rope_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swa.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE = 0, 1, 2, 3, 4
P = ctypes.c_void_p(0x10000)      # aligned fake device pointer (never dereferenced)
MIS = ctypes.c_void_p(0x10008)    # misaligned fake pointer


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \t\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from causal_sliding_window_rope_amd.build import build
        build()
    return binding.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("swa_fwd", "swa_bwd", "rope_qknorm_fwd", "rope_qknorm_bwd", "ve_gate_v",
              "ve_gate_v_bwd", "rope_table", "swa_bwd_workspace_size", "swa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(binding.SIGNATURES) == set(declared_functions())


def declared_param_kinds():
    """name -> list of 'p' (pointer), 'i' (int / enum), 'f' (float), 'd' (double), 's' (size_t)
    for every function the header declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"^[A-Za-z_][\w \t\*]*?\b([a-z_][a-z0-9_]*)\s*\(([^)]*)\)\s*;", text,
                         flags=re.M):
        params = [x.strip() for x in m.group(2).split(",") if x.strip() and x.strip() != "void"]
        kinds = []
        for prm in params:
            if "*" in prm:
                kinds.append("p")
            elif prm.startswith("size_t"):
                kinds.append("s")
            elif prm.startswith("double"):
                kinds.append("d")
            elif prm.startswith("float"):
                kinds.append("f")
            else:
                kinds.append("i")
        out[m.group(1)] = kinds
    return out


def test_binding_signatures_match_the_header():
    kinds = declared_param_kinds()
    code = {ctypes.c_void_p: "p", ctypes.c_int: "i", ctypes.c_float: "f", ctypes.c_double: "d",
            ctypes.c_size_t: "s"}
    assert set(kinds) == set(binding.SIGNATURES)
    for name, (_, args) in binding.SIGNATURES.items():
        assert [code[a] for a in args] == kinds[name], name


def _fwd(lib, q=P, k=P, v=P, ve=None, gate=None, o=P, lse=P, B=1, T=8, H=1, D=64, W=4, scale=0.125,
         dt=1, doc=None, ids=None, rows=0):
    return lib.swa_fwd(q, k, v, ve, gate, ids, rows, doc, o, lse, B, T, H, D, W, scale, dt, None)


def test_swa_fwd_validation(lib):
    assert _fwd(lib, q=None) == INVALID and b"q must not be NULL" in lib.swa_last_error()
    assert _fwd(lib, D=96) == UNSUPPORTED
    assert _fwd(lib, D=32) == UNSUPPORTED
    assert _fwd(lib, k=MIS) == ALIGN
    assert _fwd(lib, W=0) == INVALID
    assert _fwd(lib, W=-2) == INVALID
    assert _fwd(lib, scale=0.0) == INVALID
    assert _fwd(lib, scale=float("nan")) == INVALID
    assert _fwd(lib, B=0) == INVALID
    assert _fwd(lib, T=0) == INVALID
    assert _fwd(lib, dt=7) == INVALID
    assert _fwd(lib, ve=P) == INVALID          # ve without gate
    assert _fwd(lib, gate=P) == INVALID        # gate without ve
    assert _fwd(lib, B=1 << 20, T=1 << 12, H=1 << 4, D=128) == UNSUPPORTED
    assert _fwd(lib, doc=MIS) == ALIGN                     # document bounds misaligned
    # value-embedding table mode: ids need the gate, a positive row count, and rows need ids
    assert _fwd(lib, ids=P, rows=4) == INVALID
    assert _fwd(lib, ve=P, gate=P, ids=P, rows=0) == INVALID
    assert _fwd(lib, ve=P, gate=P, rows=3) == INVALID
    assert _fwd(lib, ve=P, gate=P, ids=P, rows=1 << 30, H=1 << 4, D=128) == UNSUPPORTED


def test_doc_bounds_validation(lib):
    assert lib.swa_doc_bounds(None, P, 2, 8, None) == INVALID
    assert lib.swa_doc_bounds(P, None, 2, 8, None) == INVALID
    assert lib.swa_doc_bounds(P, ctypes.c_void_p(0x20000), 0, 8, None) == INVALID
    assert lib.swa_doc_bounds(P, P, 2, 8, None) == INVALID       # output aliases the ids
    assert lib.swa_doc_bounds(P, ctypes.c_void_p(0x20008), 2, 8, None) == ALIGN


def test_swa_bwd_validation(lib):
    ws_need = lib.swa_bwd_workspace_size(2, 64, 3, 64, 1)
    assert ws_need >= 2 * (2 * 64 * 3 * 4)          # delta and lse*log2(e), float32 each
    assert lib.swa_bwd_workspace_size(2, 64, 3, 96, 1) == 0

    def bwd(ws=P, ws_bytes=ws_need, ve=None, gate=None, dve=None, dgate=None, W=8, dO=P, ids=None,
            rows=0):
        return lib.swa_bwd(P, P, P, ve, gate, ids, rows, None, P, P, dO, P, P, P, dve, dgate, ws,
                           ws_bytes, 2, 64, 3, 64, W, 0.125, 1, None)

    assert bwd(ws=None) == WORKSPACE
    assert bwd(ws_bytes=ws_need - 1) == WORKSPACE
    assert bwd(ws=ctypes.c_void_p(0x10010)) == ALIGN
    assert bwd(ve=P, gate=P) == INVALID                 # gate without dve/dgate
    assert bwd(dve=P, dgate=P) == INVALID               # dve/dgate without gate
    assert bwd(W=0) == INVALID
    assert bwd(dO=None) == INVALID
    assert bwd(ids=P, rows=5) == INVALID                 # table ids without the gate
    assert bwd(ve=P, gate=P, dve=P, dgate=P, ids=P, rows=-1) == INVALID

    # the two compute stages check the same arguments
    def dkdv(ws=P, ws_bytes=ws_need, W=8):
        return lib.swa_bwd_dkdv(P, P, P, None, None, None, 0, None, P, P, P, P, None, None, ws,
                                ws_bytes, 2, 64, 3, 64, W, 0.125, 1, None)

    def dq(ws=P, ws_bytes=ws_need, W=8, ve=None, gate=None, ids=None, rows=0):
        return lib.swa_bwd_dq(P, P, P, ve, gate, ids, rows, None, P, P, P, ws, ws_bytes, 2, 64, 3, 64,
                              W, 0.125, 1, None)

    assert dkdv(ws=None) == WORKSPACE and dq(ws=None) == WORKSPACE
    assert dkdv(ws_bytes=ws_need - 1) == WORKSPACE and dq(ws_bytes=ws_need - 1) == WORKSPACE
    assert dkdv(W=0) == INVALID and dq(W=0) == INVALID
    assert dq(ve=P) == INVALID                          # ve without gate
    assert dq(ve=P, gate=P, ids=P, rows=0) == INVALID   # table mode without rows


def test_fused_query_prologue_validation(lib):
    """swa_fwd_qnorm / swa_bwd_dq_ds_qnorm (the query half of the prologue inside the attention
    kernels) and the k-only forms of the prologue calls: host-side checks only."""
    A = ctypes.c_void_p(0x20000)

    def fwd(q=P, cs=P, eps=1e-6, qn=A, dtype=1, W=8):
        return lib.swa_fwd_qnorm(q, cs, eps, P, P, None, None, None, 0, None, qn, P, P, 2, 64, 3,
                                 64, W, 0.125, dtype, None)

    assert fwd(dtype=0) == UNSUPPORTED                 # bfloat16 only
    assert fwd(q=None) == INVALID and fwd(cs=None) == INVALID and fwd(qn=None) == INVALID
    assert fwd(eps=-1.0) == INVALID
    assert fwd(qn=P) == INVALID                        # qn aliases q
    assert fwd(W=0) == INVALID and fwd(q=MIS) == ALIGN
    nws = lib.swa_bwd_ds_workspace_size(2, 64, 3, 64, 8, 1)

    def dq(q=P, cs=P, eps=1e-6, out=A, ws_bytes=nws, dtype=1):
        return lib.swa_bwd_dq_ds_qnorm(P, None, q, cs, eps, out, P, ws_bytes, 2, 64, 3, 64, 8,
                                       0.125, dtype, None)

    assert dq(dtype=0) == UNSUPPORTED
    assert dq(q=None) == INVALID and dq(cs=None) == INVALID and dq(out=None) == INVALID
    assert dq(eps=float("nan")) == INVALID
    assert dq(out=P) == INVALID                        # dq aliases q
    assert dq(ws_bytes=nws - 1) == WORKSPACE
    # k only: q and its outputs NULL together
    assert lib.rope_qknorm_fwd(None, P, P, A, ctypes.c_void_p(0x30000), 1, 8, 1, 64, 1e-6, 1,
                               None) == INVALID       # qn without q
    assert lib.rope_qknorm_bwd(None, P, P, None, P, A, ctypes.c_void_p(0x30000), 1, 8, 1, 64,
                               1e-6, 1, None) == INVALID   # dq without q


def test_swa_bwd_noalloc_validation(lib):
    """Checks that run on the host before the scratch is touched: bad arguments, and sizes whose
    workspace would not fit the library's static scratch."""
    def call(B=1, T=64, H=2, D=64, W=16, dq=P, o=P):
        return lib.swa_bwd_noalloc(P, P, P, None, None, None, 0, None, o, P, P, dq, P, P, None,
                                   None, B, T, H, D, W, 0.125, 1, None)

    assert call(dq=None) == INVALID and call(o=None) == INVALID
    assert call(W=0) == INVALID and call(D=96) == UNSUPPORTED
    assert call(dq=MIS) == ALIGN
    rows = 2_097_024                 # the most rows whose workspace fits 16 MiB
    assert lib.swa_bwd_workspace_size(1, rows, 1, 64, 1) <= 16 << 20
    assert lib.swa_bwd_workspace_size(1, rows + 1, 1, 64, 1) > 16 << 20
    assert call(B=1, T=4096, H=1024) == WORKSPACE
    assert b"SWA_NOALLOC_SCRATCH_BYTES" in lib.swa_last_error()


def test_fp8_validation(lib):
    assert lib.swa_fp8_v_bytes(2, 100, 3, 128) == 2 * 3 * 128 * 128     # T padded to 128
    assert lib.swa_fp8_v_bytes(2, 100, 3, 96) == 0

    def pack(q=P, k=P, v=P, q8=P, k8=P, v8=P, sq=1.0, sk=1.0, sv=1.0, D=64):
        return lib.swa_fp8_pack(q, k, v, sq, sk, sv, q8, k8, v8, 1, 8, 2, D, 1, None)

    assert pack(q8=None) == INVALID                      # q without q8
    assert pack(q=None, k=None, v=None, q8=None, k8=None, v8=None) == INVALID   # nothing to do
    assert pack(sv=0.0) == INVALID and pack(sq=float("nan")) == INVALID
    assert pack(sk=1e-39) == INVALID                     # reciprocal overflows
    assert pack(v8=MIS) == ALIGN
    assert pack(D=96) == UNSUPPORTED

    def fwd(q8=P, k8=P, v8=P, sq=1.0, W=4, scale=0.125, doc=None):
        return lib.swa_fwd_fp8(q8, k8, v8, sq, 1.0, 1.0, doc, P, P, 1, 8, 2, 64, W, scale, None)

    assert fwd(q8=None) == INVALID
    assert fwd(sq=-1.0) == INVALID
    assert fwd(W=0) == INVALID and fwd(scale=0.0) == INVALID
    assert fwd(doc=MIS) == ALIGN
    assert lib.rope_qknorm_fwd_fp8(P, P, P, None, P, 1, 8, 2, 64, 1e-6, 1, None) == INVALID
    assert lib.rope_qknorm_fwd_fp8(P, P, P, P, MIS, 1, 8, 2, 64, 1e-6, 1, None) == ALIGN
    assert lib.rope_qknorm_fwd_fp8(P, P, P, P, P, 1, 8, 2, 64, -1.0, 1, None) == INVALID
    assert lib.rope_qknorm_fwd_fp8(P, P, P, P, P, 1, 8, 2, 32, 1e-6, 1, None) == UNSUPPORTED


def test_prologue_and_gate_validation(lib):
    assert lib.rope_table(None, 8, 64, 1e4, None) == INVALID
    assert lib.rope_table(P, 8, 48, 1e4, None) == UNSUPPORTED
    assert lib.rope_table(P, 8, 64, -1.0, None) == INVALID
    assert lib.rope_qknorm_fwd(P, P, P, P, P, 1, 8, 1, 64, -1.0, 1, None) == INVALID   # eps < 0
    assert lib.rope_qknorm_fwd(P, P, P, P, ctypes.c_void_p(0x20000), 1, 8, 1, 64, 1e-6, 1, None) \
        == INVALID   # qn aliases q
    assert lib.rope_qknorm_fwd(P, MIS, P, ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000), 1, 8,
                               1, 64, 1e-6, 1, None) == ALIGN
    assert lib.rope_qknorm_bwd(P, P, P, None, P, P, P, 1, 8, 1, 64, 1e-6, 1, None) == INVALID
    assert lib.ve_gate_v(P, 16, P, P, None, None, None, 0, None, 1, 8, 2, 64, 1, None) == INVALID  # ldx
    assert lib.ve_gate_v(P, 64, P, P, P, None, None, 0, None, 1, 8, 2, 64, 1, None) == INVALID  # partial
    # table ids without the materialisation, and a table without rows
    assert lib.ve_gate_v(P, 64, P, P, None, None, P, 4, None, 1, 8, 2, 64, 1, None) == INVALID
    assert lib.ve_gate_v(P, 64, P, P, P, P, P, 0, P, 1, 8, 2, 64, 1, None) == INVALID
    assert lib.ve_gate_dv(None, P, None, 0, P, P, P, 1, 8, 2, 64, 1, None) == INVALID
    assert lib.ve_gate_dv(P, P, None, 0, P, P, None, 1, 8, 2, 64, 1, None) == INVALID   # no dgate
    assert lib.ve_gate_dv(P, P, None, 3, P, P, P, 1, 8, 2, 64, 1, None) == INVALID      # rows, no ids
    assert lib.ve_gate_dv(P, P, None, 0, P, P, P, 1, 8, 2, 96, 1, None) == UNSUPPORTED
    assert lib.ve_gate_dv(P, MIS, None, 0, P, P, P, 1, 8, 2, 64, 1, None) == ALIGN
    nws = lib.ve_gate_v_bwd_workspace_size(1, 8, 2)
    assert nws == 32 * 2 * 4                               # one chunk of 128 rows
    assert lib.ve_gate_v_bwd_workspace_size(1, 300, 3) == 3 * 32 * 3 * 4
    assert lib.ve_gate_v_bwd_workspace_size(1, 8, 65) == 0
    assert lib.ve_gate_v_bwd(P, 64, P, P, None, P, None, P, nws, 1, 8, 2, 1, None) == INVALID
    assert lib.ve_gate_v_bwd(P, 64, P, P, P, P, None, None, nws, 1, 8, 2, 1, None) == WORKSPACE
    assert lib.ve_gate_v_bwd(P, 64, P, P, P, P, None, P, nws - 4, 1, 8, 2, 1, None) == WORKSPACE
    assert lib.ve_gate_v_bwd(P, 64, P, P, P, P, None, MIS, nws, 1, 8, 2, 1, None) == ALIGN
    assert lib.ve_gate_v_bwd(P, 64, P, P, P, P, None, P, nws, 1, 8, 65, 1, None) == UNSUPPORTED
    assert lib.swa_last_error()  # message is set


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 8, 1, 64)
    with pytest.raises(ValueError):
        binding.swa_fwd(x, x, x, window=4)


def test_decode_validation(lib):
    ws = lib.swa_decode_workspace_size(2, 3, 64, 16, 8)
    assert ws >= 256
    assert lib.swa_decode_workspace_size(2, 3, 64, 16, 17) == 0      # window larger than the ring
    assert lib.swa_decode_workspace_size(2, 3, 96, 16, 8) == 0

    def dec(W=8, cap=16, wsp=P, nbytes=ws, D=64, pos=P):
        return lib.swa_decode(P, P, P, pos, P, P, wsp, nbytes, 2, 3, D, cap, W, 0.125, 1, None)

    assert dec(W=17) == INVALID
    assert dec(W=0) == INVALID
    assert dec(D=96) == UNSUPPORTED
    assert dec(pos=None) == INVALID
    assert dec(wsp=None) == WORKSPACE
    assert dec(nbytes=ws - 1) == WORKSPACE
    assert dec(wsp=ctypes.c_void_p(0x10010)) == ALIGN
    assert lib.swa_decode_prologue(P, P, P, P, 0, P, P, P, P, 2, 3, 64, 16, 1e-6, 1, None) == INVALID
    assert lib.swa_decode_prologue(P, P, P, P, 8, P, P, P, P, 2, 3, 64, 0, 1e-6, 1, None) == INVALID

"""ctypes binding of libsas.so (the C ABI declared in include/sas.h).

Argument marshalling only: every computation runs in the library's HIP kernels. torch
supplies device memory and the current HIP stream. Each function carries the name of
the C entry point it calls, returns the output tensors, and raises SasError when the
library rejects the call. There is no fallback: if libsas.so is missing or fails to load,
the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

# SAS_LIB names another build of the same library (e.g. the AddressSanitizer build of
# the host layer that the CPU tests load); there is no fallback either way.
LIB_PATH = os.environ.get("SAS_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsas.so")

SAS_OK, SAS_ERR_INVALID_ARG, SAS_ERR_UNSUPPORTED, SAS_ERR_WORKSPACE, SAS_ERR_HIP = range(5)
SCOPE = {"sparse": 0, "full": 1}
GATE = {"softmax": 0, "softmax_selected": 1, "sigmoid": 2, "exp": 3}
PLACEMENT = {"inside": 0, "outside": 1}
ROWS = {"prefill": 0, "decode": 1}
BLOCK = 64

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t

SIGNATURES = {
    "sas_version": ([], ctypes.c_char_p),
    "sas_status_string": ([_I], ctypes.c_char_p),
    "sas_last_error": ([], ctypes.c_char_p),
    "sas_gates": ([_P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P], _I),
    "sas_topk_select": ([_P, _I, _I, _I, _I, _I, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P], _I),
    "sas_gates_bwd": ([_P, _I, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _I, _P, _P], _I),
    "sas_pool_keys": ([_P, _I, _I, _I, _I, _P, _I, _P, _P], _I),
    "sas_decode_early_stop": ([_P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _P, _P, _P], _I),
    "sas_decode_paged": ([_P, _P, _P, _I, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _SZ, _P], _I),
    "sas_decode_select": ([_P, _P, _I, _I, _I, _I, _I, _P, _F, _I, _I, _P, _P, _P, _P, _P, _P], _I),
    "sas_attn_fwd": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P], _I),
    "sas_attn_bwd_workspace_size": ([_I, _I, _I, _I, _I, _I, _I], _SZ),
    "sas_attn_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                      _P, _P, _P, _P, _P, _SZ, _P], _I),
    "sas_decode_workspace_size": ([_I, _I, _I, _I, _I], _SZ),
    "sas_decode": ([_P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _SZ, _P], _I),
    "sas_decode_noalloc": ([_P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P], _I),
    "sas_decode_topk": ([_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _SZ, _P], _I),
    "sas_decode_paged_topk": ([_P, _P, _P, _I, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _SZ,
                               _P], _I),
    "sas_decode_long_workspace_size": ([_I, _I, _I, _I, _I, _I], _SZ),
    "sas_decode_long": ([_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _SZ, _P], _I),
    "sas_pool_keys_paged": ([_P, _I, _P, _I, _I, _I, _I, _P, _I, _P, _P], _I),
    "sas_decode_long_paged": ([_P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _SZ,
                               _P], _I),
    "sas_profile_enable": ([_I], _I),
    "sas_profile_only": ([ctypes.c_char_p], _I),
    "sas_profile_collect": ([_I, ctypes.c_char_p, _I, _P, _P], _I),
    "sas_profile_collect_launches": ([_I, ctypes.c_char_p, _I, _P], _I),
    "sas_debug_workgroup_order": ([ctypes.c_ulonglong], _I),
    "sas_measure_mfma": ([_I, _I, _P, _P, _P], _I),
    "sas_measure_read": ([_P, _SZ, _P, _P], _I),
}


class SasError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{status_string(status)}: {detail}")


def lib():
    """Load libsas.so once and declare the C signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(or python -m learned_context_ranking_amd.build_lib)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_string(st: int) -> str:
    return lib().sas_status_string(int(st)).decode()


def version() -> str:
    return lib().sas_version().decode()


def _check(st):
    if st != SAS_OK:
        raise SasError(st, lib().sas_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ------------------------------------------------------------------ entry points

def sas_gates(s, mode="prefill", row_valid=None, cols=None, want_g=False):
    """s: fp32 [B, H, rows, ld]. Returns (lse [B, H, rows], g or None)."""
    _need(s, torch.float32, "s")
    B, H, rows, ld = s.shape
    cols = ld if cols is None else cols
    lse = torch.empty((B, H, rows), dtype=torch.float32, device=s.device)
    g = torch.empty_like(s) if want_g else None
    if row_valid is not None:
        _need(row_valid, torch.int32, "row_valid")
    _check(lib().sas_gates(_ptr(s), B, H, rows, cols, ld, ROWS[mode], _ptr(row_valid), _ptr(lse),
                           _ptr(g), _stream(s.device)))
    return lse, g


def sas_topk_select(s, topk, scope="sparse", mode="prefill", row_valid=None, kcap=None, cols=None,
                    gate="softmax"):
    """s: fp32 [B, H, rows, ld]. Returns idx int32 [B, H, rows, kcap], cnt int32 [B, H, rows],
    lse fp32 [B, H, rows] (the gate's normaliser), logg fp32 [B, H, rows, kcap]."""
    _need(s, torch.float32, "s")
    B, H, rows, ld = s.shape
    cols = ld if cols is None else cols
    if kcap is None:
        kcap = cols if scope == "full" else min(topk, cols)
    dev = s.device
    idx = torch.empty((B, H, rows, kcap), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H, rows), dtype=torch.int32, device=dev)
    lse = torch.empty((B, H, rows), dtype=torch.float32, device=dev)
    logg = torch.empty((B, H, rows, kcap), dtype=torch.float32, device=dev)
    if row_valid is not None:
        _need(row_valid, torch.int32, "row_valid")
    _check(lib().sas_topk_select(_ptr(s), B, H, rows, cols, ld, ROWS[mode], _ptr(row_valid), int(topk),
                                 SCOPE[scope], GATE[gate], kcap, _ptr(idx), _ptr(cnt), _ptr(lse), _ptr(logg),
                                 _stream(dev)))
    return idx, cnt, lse, logg


def sas_gates_bwd(s, lse, idx, cnt, dg, mode="prefill", row_valid=None, cols=None, out=None, gate="softmax"):
    """Gradient with respect to s through the gate activation.
    s fp32 [B, H, rows, ld]; lse [B, H, rows] from sas_topk_select with the same gate (may
    be None for sigmoid / exp); idx int32 and dg fp32 [B, H, rows, kcap]; cnt int32
    [B, H, rows]. Returns ds fp32 [B, H, rows, ld]."""
    _need(s, torch.float32, "s")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    _need(idx, torch.int32, "idx")
    _need(cnt, torch.int32, "cnt")
    _need(dg, torch.float32, "dg")
    B, H, rows, ld = s.shape
    kcap = idx.shape[-1]
    if tuple(idx.shape) != (B, H, rows, kcap) or tuple(dg.shape) != (B, H, rows, kcap):
        raise ValueError(f"idx {tuple(idx.shape)} / dg {tuple(dg.shape)} do not match s {tuple(s.shape)}")
    if (lse is not None and tuple(lse.shape) != (B, H, rows)) or tuple(cnt.shape) != (B, H, rows):
        raise ValueError(f"lse {tuple(lse.shape)} / cnt {tuple(cnt.shape)} do not match s {tuple(s.shape)}")
    cols = ld if cols is None else cols
    if row_valid is not None:
        _need(row_valid, torch.int32, "row_valid")
    ds = torch.empty_like(s) if out is None else out
    _need(ds, torch.float32, "out")
    _check(lib().sas_gates_bwd(_ptr(s), B, H, rows, cols, ld, ROWS[mode], _ptr(row_valid), GATE[gate], _ptr(lse),
                               _ptr(idx), _ptr(cnt), _ptr(dg), kcap, _ptr(ds), _stream(s.device)))
    return ds


def sas_attn_fwd(Q, K, V, idx, cnt, logg, scale, out=None, lse_out=None, placement="inside"):
    """Q bf16 [B, Hq, n, d]; K, V bf16 [B, Hkv, n, d]; idx/cnt/logg from sas_topk_select.
    placement: "inside" (log g in the logits) or "outside" (p g after the softmax).
    Returns (O bf16 [B, Hq, n, d], lse_rows fp32 [B, Hq, n])."""
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, torch.bfloat16, nm)
    _need(idx, torch.int32, "idx")
    _need(cnt, torch.int32, "cnt")
    if logg is not None:
        _need(logg, torch.float32, "logg")
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    kcap = idx.shape[-1]
    O = torch.empty_like(Q) if out is None else out
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device=Q.device) if lse_out is None else lse_out
    _check(lib().sas_attn_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(idx), _ptr(cnt), _ptr(logg), B, Hq, Hkv, n,
                              d, BLOCK, kcap, float(scale), PLACEMENT[placement], _ptr(O), _ptr(lse),
                              _stream(Q.device)))
    return O, lse


def bwd_workspace(B, Hq, Hkv, n, d, kcap, device):
    nbytes = lib().sas_attn_bwd_workspace_size(B, Hq, Hkv, n, d, BLOCK, kcap)
    if nbytes == 0:
        raise SasError(SAS_ERR_INVALID_ARG, "invalid sizes for sas_attn_bwd_workspace_size")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def sas_attn_bwd(Q, K, V, O, dO, lse_rows, idx, cnt, logg, scale, ws=None, outs=None, placement="inside"):
    """Returns (dQ fp32, dK fp32, dV fp32, dg fp32 [B, Hkv, n/64, kcap])."""
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V"), (O, "O"), (dO, "dO")):
        _need(t, torch.bfloat16, nm)
    _need(lse_rows, torch.float32, "lse_rows")
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    kcap = idx.shape[-1]
    dev = Q.device
    if ws is None:
        ws = bwd_workspace(B, Hq, Hkv, n, d, kcap, dev)
    if outs is None:
        dQ = torch.empty(Q.shape, dtype=torch.float32, device=dev)
        dK = torch.empty(K.shape, dtype=torch.float32, device=dev)
        dV = torch.empty(V.shape, dtype=torch.float32, device=dev)
        dg = torch.empty((B, Hkv, n // BLOCK, kcap), dtype=torch.float32, device=dev)
    else:
        dQ, dK, dV, dg = outs
    _check(lib().sas_attn_bwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(lse_rows), _ptr(idx),
                              _ptr(cnt), _ptr(logg), B, Hq, Hkv, n, d, BLOCK, kcap, float(scale),
                              PLACEMENT[placement], _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dg), _ptr(ws), ws.numel(),
                              _stream(dev)))
    return dQ, dK, dV, dg


def decode_workspace(B, Hq, Hkv, d, kcap, device):
    nbytes = lib().sas_decode_workspace_size(B, Hq, Hkv, d, kcap)
    if nbytes == 0:
        raise SasError(SAS_ERR_INVALID_ARG, "invalid sizes for sas_decode_workspace_size")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def sas_decode(q, Kc, Vc, kv_len, idx, cnt, scale, logg=None, ws=None, out=None):
    """q bf16 [B, Hq, d]; Kc, Vc bf16 [B, Hkv, Lmax, d]; kv_len int32 [B];
    idx int32 [B, Hkv, kcap] (or [B, Hkv, 1, kcap]); cnt int32 [B, Hkv(, 1)]. Returns o bf16."""
    for t, nm in ((q, "q"), (Kc, "Kc"), (Vc, "Vc")):
        _need(t, torch.bfloat16, nm)
    _need(kv_len, torch.int32, "kv_len")
    B, Hq, d = q.shape
    Hkv, Lmax = Kc.shape[1], Kc.shape[2]
    kcap = idx.shape[-1]
    if ws is None:
        ws = decode_workspace(B, Hq, Hkv, d, kcap, q.device)
    o = torch.empty_like(q) if out is None else out
    _check(lib().sas_decode(_ptr(q), _ptr(Kc), _ptr(Vc), _ptr(kv_len), Lmax, _ptr(idx), _ptr(cnt), _ptr(logg),
                            B, Hq, Hkv, d, BLOCK, kcap, float(scale), _ptr(o), _ptr(ws), ws.numel(),
                            _stream(q.device)))
    return o


def sas_decode_topk(q, Kc, Vc, kv_len, s, topk, scale, ws=None, out=None, want_idx=False):
    """One decode step with its Top-K selection in the same launch. q bf16 [B, Hq, d];
    Kc/Vc bf16 [B, Hkv, Lmax, d]; kv_len int32 [B]; s fp32 [B, Hkv, ld] history block
    scores (or [B, Hkv, 1, ld]). Returns o bf16 [B, Hq, d], and with want_idx also the kept
    blocks idx int32 [B, Hkv, topk] and cnt int32 [B, Hkv]."""
    for t, nm in ((q, "q"), (Kc, "Kc"), (Vc, "Vc")):
        _need(t, torch.bfloat16, nm)
    _need(kv_len, torch.int32, "kv_len")
    _need(s, torch.float32, "s")
    B, Hq, d = q.shape
    Hkv, Lmax = Kc.shape[1], Kc.shape[2]
    ld = s.shape[-1]
    dev = q.device
    if ws is None:
        ws = decode_workspace(B, Hq, Hkv, d, topk, dev)
    o = torch.empty_like(q) if out is None else out
    idx = cnt = None
    if want_idx:
        idx = torch.empty((B, Hkv, topk), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    _check(lib().sas_decode_topk(_ptr(q), _ptr(Kc), _ptr(Vc), _ptr(kv_len), Lmax, _ptr(s), ld, int(topk), B, Hq,
                                 Hkv, d, 64, float(scale), _ptr(o), _ptr(idx), _ptr(cnt), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(dev)))
    return (o, idx, cnt) if want_idx else o


def sas_decode_noalloc(q, Kc, Vc, kv_len, idx, cnt, scale, logg=None, out=None):
    """sas_decode without a workspace (the library's per-device scratch holds the partial
    states; calls that overlap on one device race). `out` must be given where the caller
    cannot allocate. Returns o bf16 [B, Hq, d]."""
    for t, nm in ((q, "q"), (Kc, "Kc"), (Vc, "Vc")):
        _need(t, torch.bfloat16, nm)
    _need(kv_len, torch.int32, "kv_len")
    B, Hq, d = q.shape
    Hkv, Lmax = Kc.shape[1], Kc.shape[2]
    kcap = idx.shape[-1]
    o = torch.empty_like(q) if out is None else out
    _check(lib().sas_decode_noalloc(_ptr(q), _ptr(Kc), _ptr(Vc), _ptr(kv_len), Lmax, _ptr(idx), _ptr(cnt),
                                    _ptr(logg), B, Hq, Hkv, d, BLOCK, kcap, float(scale), _ptr(o),
                                    _stream(q.device)))
    return o


def sas_decode_early_stop(q, Kc, Vc, kv_len, idx, cnt, order, scale, tau, out=None, used=None):
    """q bf16 [B, Hq, d]; Kc, Vc bf16 [B, Hkv, Lmax, d]; kv_len int32 [B]; idx int32 and order
    fp32 [B, Hkv, kcap] (kcap <= 63); cnt int32 [B, Hkv]. Returns (o bf16 [B, Hq, d],
    used int32 [B, Hq])."""
    for t, nm in ((q, "q"), (Kc, "Kc"), (Vc, "Vc")):
        _need(t, torch.bfloat16, nm)
    _need(kv_len, torch.int32, "kv_len")
    _need(order, torch.float32, "order")
    B, Hq, d = q.shape
    Hkv, Lmax = Kc.shape[1], Kc.shape[2]
    kcap = idx.shape[-1]
    o = torch.empty_like(q) if out is None else out
    u = torch.empty((B, Hq), dtype=torch.int32, device=q.device) if used is None else used
    _check(lib().sas_decode_early_stop(_ptr(q), _ptr(Kc), _ptr(Vc), _ptr(kv_len), Lmax, _ptr(idx), _ptr(cnt),
                                       _ptr(order), B, Hq, Hkv, d, BLOCK, kcap, float(scale), float(tau), _ptr(o),
                                       _ptr(u), _stream(q.device)))
    return o, u


def sas_decode_paged(q, Kpool, Vpool, page_table, kv_len, idx, cnt, scale, logg=None, ws=None, out=None):
    """q bf16 [B, Hq, d]; Kpool, Vpool bf16 [num_pages, Hkv, 64, d]; page_table int32
    [B, max_pages]; kv_len int32 [B]; idx int32 [B, Hkv, kcap]; cnt int32 [B, Hkv].
    Returns o bf16 [B, Hq, d]."""
    for t, nm in ((q, "q"), (Kpool, "Kpool"), (Vpool, "Vpool")):
        _need(t, torch.bfloat16, nm)
    _need(page_table, torch.int32, "page_table")
    _need(kv_len, torch.int32, "kv_len")
    B, Hq, d = q.shape
    num_pages, Hkv = Kpool.shape[0], Kpool.shape[1]
    if Kpool.shape[2] != BLOCK or tuple(Vpool.shape) != tuple(Kpool.shape):
        raise ValueError(f"pools must be [num_pages, Hkv, {BLOCK}, d] (got {tuple(Kpool.shape)}, {tuple(Vpool.shape)})")
    max_pages = page_table.shape[1]
    kcap = idx.shape[-1]
    if ws is None:
        ws = decode_workspace(B, Hq, Hkv, d, kcap, q.device)
    o = torch.empty_like(q) if out is None else out
    _check(lib().sas_decode_paged(_ptr(q), _ptr(Kpool), _ptr(Vpool), num_pages, _ptr(page_table), max_pages,
                                  _ptr(kv_len), _ptr(idx), _ptr(cnt), _ptr(logg), B, Hq, Hkv, d, BLOCK, kcap,
                                  float(scale), _ptr(o), _ptr(ws), ws.numel(), _stream(q.device)))
    return o


def sas_decode_paged_topk(q, Kpool, Vpool, page_table, kv_len, s, topk, scale, ws=None, out=None, want_idx=False):
    """sas_decode_topk over a paged cache: q bf16 [B, Hq, d]; Kpool, Vpool bf16
    [num_pages, Hkv, 64, d]; page_table int32 [B, max_pages]; kv_len int32 [B]; s fp32
    [B, Hkv, ld] history block scores (or [B, Hkv, 1, ld]). Returns o bf16 [B, Hq, d], and
    with want_idx also idx int32 [B, Hkv, topk] and cnt int32 [B, Hkv]."""
    for t, nm in ((q, "q"), (Kpool, "Kpool"), (Vpool, "Vpool")):
        _need(t, torch.bfloat16, nm)
    _need(page_table, torch.int32, "page_table")
    _need(kv_len, torch.int32, "kv_len")
    _need(s, torch.float32, "s")
    B, Hq, d = q.shape
    num_pages, Hkv = Kpool.shape[0], Kpool.shape[1]
    if Kpool.shape[2] != BLOCK or tuple(Vpool.shape) != tuple(Kpool.shape):
        raise ValueError(f"pools must be [num_pages, Hkv, {BLOCK}, d] (got {tuple(Kpool.shape)}, {tuple(Vpool.shape)})")
    max_pages = page_table.shape[1]
    ld = s.shape[-1]
    dev = q.device
    if ws is None:
        ws = decode_workspace(B, Hq, Hkv, d, topk, dev)
    o = torch.empty_like(q) if out is None else out
    idx = cnt = None
    if want_idx:
        idx = torch.empty((B, Hkv, topk), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    _check(lib().sas_decode_paged_topk(_ptr(q), _ptr(Kpool), _ptr(Vpool), num_pages, _ptr(page_table), max_pages,
                                       _ptr(kv_len), _ptr(s), ld, int(topk), B, Hq, Hkv, d, BLOCK, float(scale),
                                       _ptr(o), _ptr(idx), _ptr(cnt), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(dev)))
    return (o, idx, cnt) if want_idx else o


def decode_long_workspace(B, Hq, Hkv, d, C, topk, device):
    n = lib().sas_decode_long_workspace_size(B, Hq, Hkv, d, C, int(topk))
    if n == 0:
        raise ValueError(f"no decode_long layout for B={B} Hq={Hq} Hkv={Hkv} d={d} C={C} topk={topk}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def sas_decode_long(q, kbar, Kc, Vc, kv_len, topk, scale, ws=None, out=None, want_idx=False):
    """One long-context decode step (block scores over the pooled keys, Top-K, decode) in two
    launches. q bf16 [B, Hq, d]; kbar bf16 [B, Hkv, C, d] from sas_pool_keys; Kc/Vc bf16
    [B, Hkv, Lmax, d]; kv_len int32 [B]. Returns o bf16 [B, Hq, d], and with want_idx also
    idx int32 [B, Hkv, topk] and cnt int32 [B, Hkv]."""
    for t, nm in ((q, "q"), (kbar, "kbar"), (Kc, "Kc"), (Vc, "Vc")):
        _need(t, torch.bfloat16, nm)
    _need(kv_len, torch.int32, "kv_len")
    B, Hq, d = q.shape
    Hkv, Lmax = Kc.shape[1], Kc.shape[2]
    C = kbar.shape[2]
    dev = q.device
    if ws is None:
        ws = decode_long_workspace(B, Hq, Hkv, d, C, topk, dev)
    o = torch.empty_like(q) if out is None else out
    idx = cnt = None
    if want_idx:
        idx = torch.empty((B, Hkv, topk), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    _check(lib().sas_decode_long(_ptr(q), _ptr(kbar), C, _ptr(Kc), _ptr(Vc), _ptr(kv_len), Lmax, int(topk), B, Hq,
                                 Hkv, d, BLOCK, float(scale), _ptr(o), _ptr(idx), _ptr(cnt), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(dev)))
    return (o, idx, cnt) if want_idx else o


def sas_pool_keys_paged(Kpool, page_table, kv_len, first_block=0, out=None):
    """Kpool bf16 [num_pages, Hkv, 64, d]; page_table int32 [B, max_pages]; kv_len int32
    [B]. Returns kbar bf16 [B, Hkv, max_pages, d] (as sas_pool_keys)."""
    _need(Kpool, torch.bfloat16, "Kpool")
    _need(page_table, torch.int32, "page_table")
    _need(kv_len, torch.int32, "kv_len")
    num_pages, Hkv, _, d = Kpool.shape
    B, max_pages = page_table.shape
    if out is None:
        out = torch.zeros((B, Hkv, max_pages, d), dtype=torch.bfloat16, device=Kpool.device)
    _need(out, torch.bfloat16, "out")
    _check(lib().sas_pool_keys_paged(_ptr(Kpool), num_pages, _ptr(page_table), max_pages, B, Hkv, d, _ptr(kv_len),
                                     int(first_block), _ptr(out), _stream(Kpool.device)))
    return out


def sas_decode_long_paged(q, kbar, Kpool, Vpool, page_table, kv_len, topk, scale, ws=None, out=None,
                          want_idx=False):
    """sas_decode_long over a paged cache. q bf16 [B, Hq, d]; kbar bf16 [B, Hkv, max_pages, d]
    (sas_pool_keys_paged); Kpool/Vpool bf16 [num_pages, Hkv, 64, d]; page_table int32
    [B, max_pages]; kv_len int32 [B]. Returns o, and with want_idx also idx and cnt."""
    for t, nm in ((q, "q"), (kbar, "kbar"), (Kpool, "Kpool"), (Vpool, "Vpool")):
        _need(t, torch.bfloat16, nm)
    _need(page_table, torch.int32, "page_table")
    _need(kv_len, torch.int32, "kv_len")
    B, Hq, d = q.shape
    num_pages, Hkv = Kpool.shape[0], Kpool.shape[1]
    max_pages = page_table.shape[1]
    dev = q.device
    if ws is None:
        ws = decode_long_workspace(B, Hq, Hkv, d, max_pages, topk, dev)
    o = torch.empty_like(q) if out is None else out
    idx = cnt = None
    if want_idx:
        idx = torch.empty((B, Hkv, topk), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    _check(lib().sas_decode_long_paged(_ptr(q), _ptr(kbar), _ptr(Kpool), _ptr(Vpool), num_pages, _ptr(page_table),
                                       max_pages, _ptr(kv_len), int(topk), B, Hq, Hkv, d, BLOCK, float(scale),
                                       _ptr(o), _ptr(idx), _ptr(cnt), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(dev)))
    return (o, idx, cnt) if want_idx else o


def sas_pool_keys(Kc, kv_len, first_block=0, out=None):
    """Kc bf16 [B, Hkv, Lmax, d]; kv_len int32 [B]. Returns kbar bf16 [B, Hkv, Lmax // 64, d]
    (block means of the complete blocks >= first_block; other blocks of ``out`` untouched,
    zero in a new tensor)."""
    _need(Kc, torch.bfloat16, "Kc")
    _need(kv_len, torch.int32, "kv_len")
    B, Hkv, Lmax, d = Kc.shape
    if out is None:
        out = torch.zeros((B, Hkv, Lmax // BLOCK, d), dtype=torch.bfloat16, device=Kc.device)
    _need(out, torch.bfloat16, "out")
    _check(lib().sas_pool_keys(_ptr(Kc), B, Hkv, Lmax, d, _ptr(kv_len), int(first_block), _ptr(out),
                               _stream(Kc.device)))
    return out


def sas_decode_select(q, kbar, kv_len, scale, topk, kcap=None, want_lse=False, want_logg=False, s_out=None):
    """q bf16 [B, Hq, d]; kbar bf16 [B, Hkv, C, d] (sas_pool_keys); kv_len int32 [B].
    Returns (s fp32 [B, Hkv, C], idx int32 [B, Hkv, kcap], cnt int32 [B, Hkv], lse or None,
    logg or None). Entries of s past each row's history are left as they were (-inf in a
    new tensor)."""
    _need(q, torch.bfloat16, "q")
    _need(kbar, torch.bfloat16, "kbar")
    _need(kv_len, torch.int32, "kv_len")
    B, Hq, d = q.shape
    Hkv, C = kbar.shape[1], kbar.shape[2]
    kcap = min(int(topk), C) if kcap is None else int(kcap)
    dev = q.device
    s = torch.full((B, Hkv, C), float("-inf"), dtype=torch.float32, device=dev) if s_out is None else s_out
    _need(s, torch.float32, "s_out")
    idx = torch.empty((B, Hkv, kcap), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    lse = torch.empty((B, Hkv), dtype=torch.float32, device=dev) if want_lse else None
    logg = torch.empty((B, Hkv, kcap), dtype=torch.float32, device=dev) if want_logg else None
    _check(lib().sas_decode_select(_ptr(q), _ptr(kbar), B, Hq, Hkv, d, C, _ptr(kv_len), float(scale), int(topk),
                                   kcap, _ptr(s), _ptr(idx), _ptr(cnt), _ptr(lse), _ptr(logg), _stream(dev)))
    return s, idx, cnt, lse, logg


def profile_enable(on: bool = True):
    """Turn the library's per-kernel event timing on or off (measurement only)."""
    _check(lib().sas_profile_enable(1 if on else 0))


def profile_only(name: str | None = None):
    """While timing is on, bracket only the kernels called `name` (None: every kernel)."""
    _check(lib().sas_profile_only(None if name is None else name.encode()))


def profile_collect(max_kernels: int = 32, name_len: int = 32):
    """Per-kernel totals since the last collect: {name: (launches, total_ms)}, in first
    launch order. Waits for the recorded events."""
    names = ctypes.create_string_buffer(max_kernels * name_len)
    launches = (ctypes.c_int * max_kernels)()
    total = (ctypes.c_double * max_kernels)()
    n = lib().sas_profile_collect(max_kernels, names, name_len, ctypes.cast(launches, ctypes.c_void_p),
                                  ctypes.cast(total, ctypes.c_void_p))
    if n < 0:
        raise RuntimeError("sas_profile_collect: an event query failed")
    out = {}
    for i in range(n):
        nm = names.raw[i * name_len:(i + 1) * name_len].split(b"\0", 1)[0].decode()
        out[nm] = (int(launches[i]), float(total[i]))
    return out


def profile_collect_launches(max_launches: int = 4096, name_len: int = 32):
    """Every launch recorded since the last collect, in launch order: [(name, ms)]. Waits
    for the recorded events."""
    names = ctypes.create_string_buffer(max_launches * name_len)
    ms = (ctypes.c_double * max_launches)()
    n = lib().sas_profile_collect_launches(max_launches, names, name_len, ctypes.cast(ms, ctypes.c_void_p))
    if n < 0:
        raise RuntimeError("sas_profile_collect_launches: an event query failed")
    return [(names.raw[i * name_len:(i + 1) * name_len].split(b"\0", 1)[0].decode(), float(ms[i]))
            for i in range(n)]


def measure_mfma(workgroups, iters, clocks, sink, stream=None):
    """Launch the bf16 MFMA loop (sas_measure_mfma) on the current stream; clocks is a
    device int64 tensor of 2 * workgroups entries, sink a device float tensor."""
    dev = clocks.device
    _check(lib().sas_measure_mfma(int(workgroups), int(iters), _ptr(clocks), _ptr(sink),
                                  _stream(dev) if stream is None else stream))


def measure_read(buf, sink):
    """One streaming read of the whole of `buf` (sas_measure_read) on the current stream."""
    _check(lib().sas_measure_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(buf.device)))


def debug_workgroup_order(seed: int = 0):
    """Permute the order in which the attention and decode kernels take their work items
    (seed != 0), or restore the natural order (seed 0). A debugging aid."""
    _check(lib().sas_debug_workgroup_order(int(seed)))

"""CPU checks of the C ABI: the library loads, exports every entry point declared in
include/sas.h, and rejects bad arguments with a status code before touching the device.

No call here passes valid arguments, so no kernel is ever launched: every rejected call
returns from the host-side checks, which run before any HIP call.
"""
import ctypes
import os
import re

import pytest

from learned_context_ranking_amd import sas

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sas.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sas.LIB_PATH), reason="libsas.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sas_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 29, names
    L = ctypes.CDLL(sas.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(sas.SIGNATURES)


def test_version_and_status_strings():
    assert "gfx950" in sas.version()
    assert sas.status_string(0) == "SAS_OK"
    assert sas.status_string(3) == "SAS_ERR_WORKSPACE"


FAKE = ctypes.c_void_p(0x10000)      # 16-byte aligned, never dereferenced
MIS = ctypes.c_void_p(0x10002)       # misaligned
NULL = None


def _fwd(**kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, idx=FAKE, cnt=FAKE, logg=FAKE, B=1, Hq=4, Hkv=2, n=256, d=128,
             block=64, kcap=4, scale=0.125, placement=0, O=FAKE, lse=FAKE, stream=NULL)
    a.update(kw)
    return sas.lib().sas_attn_fwd(a["Q"], a["K"], a["V"], a["idx"], a["cnt"], a["logg"], a["B"], a["Hq"],
                                  a["Hkv"], a["n"], a["d"], a["block"], a["kcap"], a["scale"], a["placement"],
                                  a["O"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Q=NULL), sas.SAS_ERR_INVALID_ARG),
    (dict(cnt=NULL), sas.SAS_ERR_INVALID_ARG),
    (dict(Hq=3), sas.SAS_ERR_INVALID_ARG),
    (dict(block=32), sas.SAS_ERR_UNSUPPORTED),
    (dict(n=100), sas.SAS_ERR_INVALID_ARG),
    (dict(d=96), sas.SAS_ERR_UNSUPPORTED),
    (dict(kcap=-1), sas.SAS_ERR_INVALID_ARG),
    (dict(scale=0.0), sas.SAS_ERR_INVALID_ARG),
    (dict(scale=float("nan")), sas.SAS_ERR_INVALID_ARG),
    (dict(scale=1e-35), sas.SAS_ERR_INVALID_ARG),
    (dict(n=1 << 24), sas.SAS_ERR_UNSUPPORTED),          # n * d * 2 bytes >= 2^31
    (dict(K=MIS), sas.SAS_ERR_INVALID_ARG),
    (dict(O=NULL), sas.SAS_ERR_INVALID_ARG),
    (dict(B=0), sas.SAS_ERR_INVALID_ARG),
    (dict(placement=2), sas.SAS_ERR_INVALID_ARG),
    (dict(placement=-1), sas.SAS_ERR_INVALID_ARG),
])
def test_fwd_rejects(kw, code):
    assert _fwd(**kw) == code
    assert sas.lib().sas_last_error().decode() != ""


def test_select_rejects():
    L = sas.lib()
    # s, B, H, rows, cols, ld, mode, row_valid, topk, scope, gate, kcap, idx, cnt, lse, logg, stream
    args = [FAKE, 1, 2, 16, 16, 16, sas.ROWS["prefill"], NULL, 4, 0, 0, 4, FAKE, FAKE, FAKE, FAKE, NULL]
    bad = list(args); bad[0] = NULL
    assert L.sas_topk_select(*bad) == sas.SAS_ERR_INVALID_ARG
    for gate in (-1, 4):
        bad = list(args); bad[10] = gate
        assert L.sas_topk_select(*bad) == sas.SAS_ERR_INVALID_ARG
    bad = list(args); bad[11] = 3          # kcap < topk
    assert L.sas_topk_select(*bad) == sas.SAS_ERR_INVALID_ARG
    bad = list(args); bad[9] = 1           # full scope needs kcap >= rows - 1 = 15
    assert L.sas_topk_select(*bad) == sas.SAS_ERR_INVALID_ARG
    bad = list(args); bad[6] = sas.ROWS["decode"]   # decode needs row_valid
    assert L.sas_topk_select(*bad) == sas.SAS_ERR_INVALID_ARG
    bad = list(args); bad[7] = FAKE        # prefill forbids row_valid
    assert L.sas_topk_select(*bad) == sas.SAS_ERR_INVALID_ARG
    bad = list(args); bad[4] = 10          # prefill: cols >= rows - 1
    assert L.sas_topk_select(*bad) == sas.SAS_ERR_INVALID_ARG
    bad = list(args); bad[4] = 9000; bad[5] = 9000
    assert L.sas_topk_select(*bad) == sas.SAS_ERR_UNSUPPORTED
    bad = list(args); bad[8] = -1
    assert L.sas_topk_select(*bad) == sas.SAS_ERR_INVALID_ARG
    g = [FAKE, 1, 2, 16, 16, 16, sas.ROWS["prefill"], NULL, NULL, NULL, NULL]
    assert L.sas_gates(*g) == sas.SAS_ERR_INVALID_ARG   # lse NULL


def test_gates_bwd_rejects():
    L = sas.lib()
    # s, B, H, rows, cols, ld, mode, row_valid, gate, lse, idx, cnt, dg, kcap, ds, stream
    args = [FAKE, 1, 2, 16, 16, 16, sas.ROWS["prefill"], NULL, 0, FAKE, FAKE, FAKE, FAKE, 4,
            ctypes.c_void_p(0x20000), NULL]
    for i, code in ((0, sas.SAS_ERR_INVALID_ARG), (9, sas.SAS_ERR_INVALID_ARG), (11, sas.SAS_ERR_INVALID_ARG),
                    (14, sas.SAS_ERR_INVALID_ARG), (10, sas.SAS_ERR_INVALID_ARG), (12, sas.SAS_ERR_INVALID_ARG)):
        bad = list(args); bad[i] = NULL
        assert L.sas_gates_bwd(*bad) == code, i
    for gate in (-1, 4):
        bad = list(args); bad[8] = gate
        assert L.sas_gates_bwd(*bad) == sas.SAS_ERR_INVALID_ARG
    bad = list(args); bad[14] = FAKE        # ds aliases s
    assert L.sas_gates_bwd(*bad) == sas.SAS_ERR_INVALID_ARG
    bad = list(args); bad[13] = 8193
    assert L.sas_gates_bwd(*bad) == sas.SAS_ERR_INVALID_ARG
    bad = list(args); bad[6] = sas.ROWS["decode"]   # decode needs row_valid
    assert L.sas_gates_bwd(*bad) == sas.SAS_ERR_INVALID_ARG
    bad = list(args); bad[4] = 9000; bad[5] = 9000
    assert L.sas_gates_bwd(*bad) == sas.SAS_ERR_UNSUPPORTED
    bad = list(args); bad[13] = -1
    assert L.sas_gates_bwd(*bad) == sas.SAS_ERR_INVALID_ARG
    assert "kcap" in L.sas_last_error().decode()


def test_pool_and_decode_select_reject():
    L = sas.lib()
    # Kc, B, Hkv, Lmax, d, kv_len, first_block, kbar, stream
    pool = [FAKE, 1, 2, 640, 128, FAKE, 0, FAKE, NULL]
    assert L.sas_pool_keys(*[NULL] + pool[1:]) == sas.SAS_ERR_INVALID_ARG
    for i, v, code in ((3, 600, sas.SAS_ERR_INVALID_ARG), (4, 96, sas.SAS_ERR_UNSUPPORTED),
                       (6, 11, sas.SAS_ERR_INVALID_ARG), (6, -1, sas.SAS_ERR_INVALID_ARG),
                       (7, MIS, sas.SAS_ERR_INVALID_ARG), (1, 0, sas.SAS_ERR_INVALID_ARG)):
        bad = list(pool); bad[i] = v
        assert L.sas_pool_keys(*bad) == code, (i, v)
    # q, kbar, B, Hq, Hkv, d, C, kv_len, scale, topk, kcap, s, idx, cnt, lse, logg, stream
    sel = [FAKE, FAKE, 2, 8, 2, 128, 8192, FAKE, 0.088, 32, 32, FAKE, FAKE, FAKE, NULL, NULL, NULL]
    for i, v, code in ((0, NULL, sas.SAS_ERR_INVALID_ARG), (11, NULL, sas.SAS_ERR_INVALID_ARG),
                       (12, NULL, sas.SAS_ERR_INVALID_ARG), (13, NULL, sas.SAS_ERR_INVALID_ARG),
                       (3, 7, sas.SAS_ERR_INVALID_ARG), (5, 80, sas.SAS_ERR_UNSUPPORTED),
                       (6, 8193, sas.SAS_ERR_UNSUPPORTED), (6, 0, sas.SAS_ERR_INVALID_ARG),
                       (9, -1, sas.SAS_ERR_INVALID_ARG), (10, 31, sas.SAS_ERR_INVALID_ARG),
                       (8, 0.0, sas.SAS_ERR_INVALID_ARG), (8, float("inf"), sas.SAS_ERR_INVALID_ARG),
                       (1, MIS, sas.SAS_ERR_INVALID_ARG)):
        bad = list(sel); bad[i] = v
        assert L.sas_decode_select(*bad) == code, (i, v)
    bad = list(sel); bad[6] = 16; bad[10] = 16     # kcap >= min(topk, C) = 16 is enough
    bad[12] = NULL
    assert L.sas_decode_select(*bad) == sas.SAS_ERR_INVALID_ARG   # idx NULL with kcap > 0


def test_bwd_workspace_and_rejects():
    L = sas.lib()
    assert L.sas_attn_bwd_workspace_size(1, 4, 2, 256, 128, 64, 4) > 0
    assert L.sas_attn_bwd_workspace_size(1, 4, 2, 250, 128, 64, 4) == 0
    assert L.sas_attn_bwd_workspace_size(1, 3, 2, 256, 128, 64, 4) == 0
    need = L.sas_attn_bwd_workspace_size(1, 4, 2, 256, 128, 64, 4)
    args = [FAKE] * 9 + [1, 4, 2, 256, 128, 64, 4, 0.125, 0] + [FAKE] * 4 + [FAKE, need - 1, NULL]
    assert L.sas_attn_bwd(*args) == sas.SAS_ERR_WORKSPACE
    args[-3] = NULL
    args[-2] = need
    assert L.sas_attn_bwd(*args) == sas.SAS_ERR_WORKSPACE
    args[-3] = FAKE
    args[4] = NULL                          # dO
    assert L.sas_attn_bwd(*args) == sas.SAS_ERR_INVALID_ARG
    args[4] = FAKE
    args[17] = 5                            # placement
    assert L.sas_attn_bwd(*args) == sas.SAS_ERR_INVALID_ARG
    # one KV group's query rows must stay below 2^31 bytes: 8 heads x 2^20 rows x 128 x 2
    big = [FAKE] * 9 + [1, 8, 1, 1 << 20, 128, 64, 4, 0.125, 0] + [FAKE] * 4 + [FAKE, 1 << 62, NULL]
    assert L.sas_attn_bwd(*big) == sas.SAS_ERR_UNSUPPORTED


def test_decode_rejects():
    L = sas.lib()
    need = L.sas_decode_workspace_size(2, 8, 2, 128, 4)
    assert need > 0
    args = [FAKE, FAKE, FAKE, FAKE, 1024, FAKE, FAKE, NULL, 2, 8, 2, 128, 64, 4, 0.1, FAKE, FAKE, need, NULL]
    bad = list(args); bad[-2] = need - 1
    assert L.sas_decode(*bad) == sas.SAS_ERR_WORKSPACE
    bad = list(args); bad[9] = 66; bad[10] = 2    # G = 33 > 32 query columns
    assert L.sas_decode(*bad) == sas.SAS_ERR_UNSUPPORTED
    bad = list(args); bad[4] = 1 << 23            # Lmax * d * 2 = 2^31
    assert L.sas_decode(*bad) == sas.SAS_ERR_UNSUPPORTED
    bad = list(args); bad[3] = NULL               # kv_len
    assert L.sas_decode(*bad) == sas.SAS_ERR_INVALID_ARG
    bad = list(args); bad[12] = 128               # block
    assert L.sas_decode(*bad) == sas.SAS_ERR_UNSUPPORTED


def test_decode_noalloc_rejects():
    """The allocation-free decode shares sas_decode's checks and rejects sizes whose launch
    would need more partial-state bytes than its 16 MiB per-device scratch (before any HIP
    call)."""
    L = sas.lib()
    # q, Kc, Vc, kv_len, Lmax, idx, cnt, logg, B, Hq, Hkv, d, block, kcap, scale, o, stream
    args = [FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE, NULL, 2, 8, 2, 128, 64, 16, 0.1, FAKE, NULL]
    for i, v, code in ((0, NULL, sas.SAS_ERR_INVALID_ARG), (3, NULL, sas.SAS_ERR_INVALID_ARG),
                       (12, 128, sas.SAS_ERR_UNSUPPORTED), (11, 96, sas.SAS_ERR_UNSUPPORTED),
                       (9, 7, sas.SAS_ERR_INVALID_ARG), (15, MIS, sas.SAS_ERR_INVALID_ARG),
                       (14, 0.0, sas.SAS_ERR_INVALID_ARG)):
        bad = list(args); bad[i] = v
        assert L.sas_decode_noalloc(*bad) == code, (i, v)
    # 511 pairs x 32 heads x d = 128 split in 2 chunks: 511 * 2 * 32 * 130 * 4 B > 16 MiB
    big = list(args); big[8] = 511; big[9] = 32; big[10] = 1; big[13] = 3
    assert L.sas_decode_noalloc(*big) == sas.SAS_ERR_UNSUPPORTED
    assert b"scratch" in L.sas_last_error()
    # 512 pairs keep one chunk per list: no partial states, accepted by the checks (the
    # call then needs a device, so it is not made here)


def test_decode_topk_rejects():
    """The decode with its own selection checks its sizes before any HIP call: K above 64
    and rows of more than 1024 history blocks are left to sas_topk_select + sas_decode."""
    L = sas.lib()
    need = L.sas_decode_workspace_size(2, 8, 2, 128, 16)
    # q, Kc, Vc, kv_len, Lmax, s, ld, topk, B, Hq, Hkv, d, block, scale, o, idx, cnt, ws, ws_bytes, stream
    args = [FAKE, FAKE, FAKE, FAKE, 4096, FAKE, 64, 16, 2, 8, 2, 128, 64, 0.1, FAKE, NULL, NULL, FAKE, need, NULL]
    for i, v, code in ((5, NULL, sas.SAS_ERR_INVALID_ARG),         # no scores
                       (7, 0, sas.SAS_ERR_INVALID_ARG),            # K = 0
                       (7, 65, sas.SAS_ERR_UNSUPPORTED),           # K above 64
                       (4, 65665, sas.SAS_ERR_UNSUPPORTED),        # 1025 history blocks
                       (6, 62, sas.SAS_ERR_INVALID_ARG),           # ld below (Lmax - 1) / 64
                       (15, FAKE, sas.SAS_ERR_INVALID_ARG),        # idx without cnt
                       (0, NULL, sas.SAS_ERR_INVALID_ARG),         # no q
                       (12, 32, sas.SAS_ERR_UNSUPPORTED),          # block != 64
                       (18, need - 1, sas.SAS_ERR_WORKSPACE)):     # workspace too small
        bad = list(args); bad[i] = v
        assert L.sas_decode_topk(*bad) == code, (i, v)


def test_decode_paged_rejects():
    L = sas.lib()
    need = L.sas_decode_workspace_size(2, 8, 2, 128, 4)
    # q, Kpool, Vpool, num_pages, page_table, max_pages, kv_len, idx, cnt, logg, B, Hq, Hkv, d, block,
    # kcap, scale, o, ws, ws_bytes, stream
    args = [FAKE, FAKE, FAKE, 100, FAKE, 16, FAKE, FAKE, FAKE, NULL, 2, 8, 2, 128, 64, 4, 0.1, FAKE, FAKE, need, NULL]
    for i, v, code in ((4, NULL, sas.SAS_ERR_INVALID_ARG), (3, 0, sas.SAS_ERR_INVALID_ARG),
                       (5, 0, sas.SAS_ERR_INVALID_ARG), (14, 32, sas.SAS_ERR_UNSUPPORTED),
                       (13, 96, sas.SAS_ERR_UNSUPPORTED), (11, 9, sas.SAS_ERR_INVALID_ARG),
                       (1, MIS, sas.SAS_ERR_INVALID_ARG), (19, need - 1, sas.SAS_ERR_WORKSPACE),
                       (16, -1.0, sas.SAS_ERR_INVALID_ARG), (7, NULL, sas.SAS_ERR_INVALID_ARG),
                       (11, 66, sas.SAS_ERR_UNSUPPORTED), (5, 1 << 25, sas.SAS_ERR_UNSUPPORTED)):
        bad = list(args); bad[i] = v      # Hq = 66 over Hkv = 2 is a group of 33 > 32
        assert L.sas_decode_paged(*bad) == code, (i, v)


def test_decode_paged_topk_rejects():
    """The paged decode with its own selection: the paged checks plus those of the
    selection (K in [1, 64], at most 1024 history blocks, ld, idx and cnt together)."""
    L = sas.lib()
    need = L.sas_decode_workspace_size(2, 8, 2, 128, 16)
    # q, Kpool, Vpool, num_pages, page_table, max_pages, kv_len, s, ld, topk, B, Hq, Hkv, d,
    # block, scale, o, idx, cnt, ws, ws_bytes, stream
    args = [FAKE, FAKE, FAKE, 100, FAKE, 64, FAKE, FAKE, 64, 16, 2, 8, 2, 128, 64, 0.1, FAKE, NULL, NULL, FAKE,
            need, NULL]
    for i, v, code in ((7, NULL, sas.SAS_ERR_INVALID_ARG),         # no scores
                       (9, 0, sas.SAS_ERR_INVALID_ARG),            # K = 0
                       (9, 65, sas.SAS_ERR_UNSUPPORTED),           # K above 64
                       (5, 1026, sas.SAS_ERR_UNSUPPORTED),         # 1025 history blocks
                       (8, 62, sas.SAS_ERR_INVALID_ARG),           # ld below max_pages - 1
                       (17, FAKE, sas.SAS_ERR_INVALID_ARG),        # idx without cnt
                       (4, NULL, sas.SAS_ERR_INVALID_ARG),         # no page table
                       (3, 0, sas.SAS_ERR_INVALID_ARG),            # no pages
                       (14, 32, sas.SAS_ERR_UNSUPPORTED),          # block != 64
                       (1, MIS, sas.SAS_ERR_INVALID_ARG),          # misaligned pool
                       (20, need - 1, sas.SAS_ERR_WORKSPACE)):     # workspace too small
        bad = list(args); bad[i] = v
        assert L.sas_decode_paged_topk(*bad) == code, (i, v)
    ok = list(args); ok[5] = 1025; ok[8] = 1024          # 1024 history blocks: accepted up to the launch
    ok[0] = NULL                                        # (then stopped by the missing q, before any HIP call)
    assert L.sas_decode_paged_topk(*ok) == sas.SAS_ERR_INVALID_ARG


def test_decode_long_rejects():
    """The two-launch long-context decode checks its sizes before any HIP call, and its
    workspace query is 0 for the sizes it rejects."""
    L = sas.lib()
    assert L.sas_decode_long_workspace_size(2, 8, 2, 128, 8192, 16) > 0
    for bad in ((2, 8, 2, 128, 8193, 16), (2, 8, 2, 128, 512, 65), (2, 8, 2, 128, 512, 0),
                (2, 8, 3, 128, 512, 16), (2, 8, 2, 96, 512, 16), (0, 8, 2, 128, 512, 16)):
        assert L.sas_decode_long_workspace_size(*bad) == 0, bad
    need = L.sas_decode_long_workspace_size(2, 8, 2, 128, 512, 16)
    # q, kbar, C, Kc, Vc, kv_len, Lmax, topk, B, Hq, Hkv, d, block, scale, o, idx, cnt, ws, ws_bytes, stream
    args = [FAKE, FAKE, 512, FAKE, FAKE, FAKE, 32768, 16, 2, 8, 2, 128, 64, 0.1, FAKE, NULL, NULL, FAKE, need, NULL]
    for i, v, code in ((1, NULL, sas.SAS_ERR_INVALID_ARG),          # no pooled keys
                       (1, MIS, sas.SAS_ERR_INVALID_ARG),           # misaligned pooled keys
                       (7, 0, sas.SAS_ERR_INVALID_ARG),             # K = 0
                       (7, 65, sas.SAS_ERR_UNSUPPORTED),            # K above 64
                       (2, 8193, sas.SAS_ERR_UNSUPPORTED),          # more than 8192 pooled blocks
                       (6, 32834, sas.SAS_ERR_INVALID_ARG),         # 513 history blocks, C = 512
                       (15, FAKE, sas.SAS_ERR_INVALID_ARG),         # idx without cnt
                       (0, NULL, sas.SAS_ERR_INVALID_ARG),          # no q
                       (12, 32, sas.SAS_ERR_UNSUPPORTED),           # block != 64
                       (18, need - 1, sas.SAS_ERR_WORKSPACE)):      # workspace too small
        bad = list(args); bad[i] = v
        assert L.sas_decode_long(*bad) == code, (i, v)
    ok = list(args); ok[6] = 32832; ok[0] = NULL     # 512 history blocks fit C = 512 (then the
    assert L.sas_decode_long(*ok) == sas.SAS_ERR_INVALID_ARG   # missing q stops it, before any HIP call)


def test_paged_long_decode_rejects():
    L = sas.lib()
    need = L.sas_decode_long_workspace_size(2, 8, 2, 128, 512, 16)
    # q, kbar, Kpool, Vpool, num_pages, page_table, max_pages, kv_len, topk, B, Hq, Hkv, d, block,
    # scale, o, idx, cnt, ws, ws_bytes, stream
    args = [FAKE, FAKE, FAKE, FAKE, 100, FAKE, 512, FAKE, 16, 2, 8, 2, 128, 64, 0.1, FAKE, NULL, NULL, FAKE, need, NULL]
    for i, v, code in ((1, NULL, sas.SAS_ERR_INVALID_ARG), (8, 65, sas.SAS_ERR_UNSUPPORTED),
                       (6, 8193, sas.SAS_ERR_UNSUPPORTED), (5, NULL, sas.SAS_ERR_INVALID_ARG),
                       (4, 0, sas.SAS_ERR_INVALID_ARG), (16, FAKE, sas.SAS_ERR_INVALID_ARG),
                       (13, 32, sas.SAS_ERR_UNSUPPORTED), (19, need - 1, sas.SAS_ERR_WORKSPACE)):
        bad = list(args); bad[i] = v
        assert L.sas_decode_long_paged(*bad) == code, (i, v)
    # Kpool, num_pages, page_table, max_pages, B, Hkv, d, kv_len, first_block, kbar, stream
    pargs = [FAKE, 100, FAKE, 512, 2, 2, 128, FAKE, 0, FAKE, NULL]
    for i, v, code in ((2, NULL, sas.SAS_ERR_INVALID_ARG), (1, 0, sas.SAS_ERR_INVALID_ARG),
                       (6, 96, sas.SAS_ERR_UNSUPPORTED), (3, 8193, sas.SAS_ERR_UNSUPPORTED),
                       (8, 513, sas.SAS_ERR_INVALID_ARG), (9, MIS, sas.SAS_ERR_INVALID_ARG)):
        bad = list(pargs); bad[i] = v
        assert L.sas_pool_keys_paged(*bad) == code, (i, v)


def test_decode_early_stop_rejects():
    L = sas.lib()
    # q, Kc, Vc, kv_len, Lmax, idx, cnt, order, B, Hq, Hkv, d, block, kcap, scale, tau, o, used, stream
    args = [FAKE, FAKE, FAKE, FAKE, 1024, FAKE, FAKE, FAKE, 2, 8, 2, 128, 64, 16, 0.1, 0.01, FAKE, NULL, NULL]
    for i, v, code in ((7, NULL, sas.SAS_ERR_INVALID_ARG), (13, 64, sas.SAS_ERR_UNSUPPORTED),
                       (15, -0.5, sas.SAS_ERR_INVALID_ARG), (15, float("nan"), sas.SAS_ERR_INVALID_ARG),
                       (12, 32, sas.SAS_ERR_UNSUPPORTED), (9, 7, sas.SAS_ERR_INVALID_ARG),
                       (16, NULL, sas.SAS_ERR_INVALID_ARG), (14, 0.0, sas.SAS_ERR_INVALID_ARG)):
        bad = list(args); bad[i] = v
        assert L.sas_decode_early_stop(*bad) == code, (i, v)


def test_profile_toggle_without_gpu():
    """Enabling and collecting the kernel timing makes no HIP call while nothing ran."""
    L = sas.lib()
    assert L.sas_profile_enable(1) == sas.SAS_OK
    assert sas.profile_collect() == {}
    assert L.sas_profile_enable(0) == sas.SAS_OK


def test_profile_only_names():
    """The one-kernel filter takes a name of up to 31 characters; NULL clears it."""
    L = sas.lib()
    assert L.sas_profile_only(b"dkv") == sas.SAS_OK
    assert L.sas_profile_only(b"x" * 31) == sas.SAS_OK
    assert L.sas_profile_only(b"x" * 32) == sas.SAS_ERR_INVALID_ARG
    assert L.sas_profile_only(None) == sas.SAS_OK

"""GPU parity of sas_attn_fwd / sas_attn_bwd against the oracle.

Small cases are compared element by element on every output (O, LSE, dQ, dK, dV, dg);
they span several query blocks, GQA groups of 1, 3, 4, 5 and 8 heads, d = 64 and 128,
full and sparse scope, ungated attention, rows whose budget exceeds their history and
the first block (no history). Full-size cases sample query blocks (O, LSE, dQ, dg are
local to a query block) and key blocks (dK, dV through the oracle's inverse map), and
check gradient invariants on every element.
"""
import numpy as np
import pytest
import torch

import oracle
from learned_context_ranking_amd import sas
from gpu_util import Prefill, assert_close, dev, host, log

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, n, d, topk, scope, gated, scores
    (1, 1, 1, 1024, 64, 4, "sparse", True, "normal"),      # the tiny oracle workload
    (1, 8, 2, 1024, 128, 4, "sparse", True, "normal"),
    (2, 8, 2, 512, 64, 3, "sparse", True, "normal"),
    (1, 10, 2, 768, 128, 6, "sparse", True, "zipf"),        # G = 5 (head split 3 + 2)
    (1, 8, 1, 512, 64, 5, "sparse", True, "planted"),       # G = 8 (two workgroups of 4)
    (1, 3, 1, 640, 128, 4, "sparse", True, "normal"),       # G = 3
    (1, 4, 1, 512, 128, 0, "full", True, "normal"),         # full scope
    (1, 4, 2, 512, 128, 4, "sparse", False, "normal"),      # ungated (logg = NULL)
    (3, 4, 1, 512, 128, 4, "sparse", True, "normal"),       # 3 (batch, KV head) pairs: odd launch phase
    (1, 4, 1, 512, 128, 0, "sparse", True, "normal"),       # budget 0: the causal current block only
    (1, 8, 2, 4096, 64, 8, "sparse", True, "zipf"),         # popular key blocks: split key-major lists
    (1, 5, 1, 4096, 128, 8, "sparse", True, "zipf"),        # the same with G = 5
    (1, 16, 1, 512, 64, 3, "sparse", True, "normal"),       # G = 16 (eight workgroups of 2 heads)
    (1, 8, 1, 512, 128, 5, "sparse", True, "planted"),      # the d = 128 forward at G = 8
    (1, 6, 2, 768, 128, 5, "sparse", True, "zipf"),         # G = 3 at d = 128 (a split with one head)
]


def _key_major_splits(idx_r, cnt_r, G):
    """Whether the key-major pass cuts some key block's list into several workgroups, by
    its planning rule: items_m = (uses_m + 1) * G; the segment length T is the smallest
    length >= 64 whose extra segments fit min(128, max(4, 4096 // (B * Hkv))) partial slots
    per (batch, KV head)."""
    B, Hkv, NB = cnt_r.shape
    budget = max(4, min(128, 4096 // (B * Hkv)))
    split = False
    for b in range(B):
        for h in range(Hkv):
            uses = np.zeros(NB, np.int64)
            for j in range(NB):
                for m in idx_r[b, h, j, :cnt_r[b, h, j]]:
                    uses[m] += 1
            items = (uses + 1) * G
            lo, hi = 64, max(64, int(items.max()))
            while lo < hi:
                mid = (lo + hi) // 2
                if int(((items + mid - 1) // mid - 1).sum()) <= budget:
                    hi = mid
                else:
                    lo = mid + 1
            split |= bool((items > lo).any())
    return split


def _run(case, seed=0, scale=None):
    B, Hq, Hkv, n, d, topk, scope, gated, scores = case
    P = Prefill(B, Hq, Hkv, n, d, seed=seed, scores=scores)
    if scale is not None:
        P.scale = scale
    t = P.device()
    NB = P.NB
    kcap = NB - 1 if scope == "full" else topk
    idx, cnt, _, logg = sas.sas_topk_select(t["s"], topk, scope=scope, kcap=kcap, cols=NB)
    lg = logg if gated else None
    O, lse = sas.sas_attn_fwd(t["Q"], t["K"], t["V"], idx, cnt, lg, P.scale)
    dQ, dK, dV, dg = sas.sas_attn_bwd(t["Q"], t["K"], t["V"], O, t["dO"], lse, idx, cnt, lg, P.scale)
    torch.cuda.synchronize()
    return P, dict(idx=idx, cnt=cnt, logg=logg, O=O, lse=lse, dQ=dQ, dK=dK, dV=dV, dg=dg), gated, scope, topk


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}-{c[2]}n{c[3]}d{c[4]}K{c[5]}{c[6]}{'' if c[7] else '-ungated'}"
                                             for c in CASES])
def test_fwd_bwd_parity(case, scale=None, grad_scale_aware=False):
    log(f"fwd/bwd parity {case}" + ("" if scale is None else f" scale={scale}"))
    P, g, gated, scope, topk = _run(case, scale=scale)
    idx_r, cnt_r, _, logg_r = oracle.select_prefill(P.s, topk, full_scope=scope == "full",
                                                    kcap=g["idx"].shape[-1])
    assert np.array_equal(host(g["idx"]), idx_r) and np.array_equal(host(g["cnt"]), cnt_r)
    if case[8] == "zipf" and case[3] >= 4096:
        assert _key_major_splits(idx_r, cnt_r, case[1] // case[2]), "case meant to split key-major lists"
    lg = logg_r if gated else np.zeros_like(logg_r)
    Q, K, V, dO = P.f32("q"), P.f32("k"), P.f32("v"), P.f32("do")
    O_r, lse_r = oracle.attn_fwd(Q, K, V, idx_r, cnt_r, lg, P.scale)
    assert_close("O", host(g["O"]), O_r)
    assert_close("LSE", host(g["lse"]), lse_r)
    dQ_r, dK_r, dV_r, dg_r = oracle.attn_bwd(Q, K, V, dO, idx_r, cnt_r, lg, P.scale)
    assert_close("dQ", host(g["dQ"]), dQ_r, scale_aware=grad_scale_aware)
    assert_close("dK", host(g["dK"]), dK_r, scale_aware=grad_scale_aware)
    assert_close("dV", host(g["dV"]), dV_r, scale_aware=grad_scale_aware)
    assert_close("dg", host(g["dg"]), dg_r, scale_aware=True)


def test_key_major_small_budget():
    """128 (batch, KV head) pairs leave 32 partial slots per pair (the budget shrinks as
    the pairs grow); with G = 8 the popular Zipf blocks still get cut. Every output against
    the oracle."""
    case = (16, 64, 8, 1024, 64, 8, "sparse", True, "zipf")
    P = Prefill(*case[:5], seed=0, scores="zipf")
    idx_r, cnt_r, _, _ = oracle.select_prefill(P.s, case[5])
    assert max(4, min(128, 4096 // (case[0] * case[2]))) == 32
    assert _key_major_splits(idx_r, cnt_r, case[1] // case[2])
    # G = 8 and Zipf-popular key blocks: a block's dK / dV sum ~7,700 query rows, so the
    # reference reaches |dK| ~ 9, |dV| ~ 15 (bf16 operands give ~0.3 % of that); the
    # gradients take the bound relative to their magnitude here
    test_fwd_bwd_parity(case, grad_scale_aware=True)


def test_fwd_bwd_group_16_d128():
    """G = 16 at d = 128 (the forward's head split: eight workgroups of two heads). Each key
    block's dV sums 16 heads x 64 rows per item, so the reference reaches |dV| ~ 10 and the
    gradients take the bound relative to their magnitude (bf16 operands give ~0.2 % of it);
    O and LSE keep the fixed bound."""
    test_fwd_bwd_parity((1, 16, 1, 512, 128, 3, "sparse", True, "normal"), grad_scale_aware=True)


@pytest.mark.parametrize("scale", [1.0, 0.02])
def test_fwd_bwd_other_scales(scale):
    """Logit scales other than 1/sqrt(d): the backward's key-major pass starts its score
    accumulators at -LSE/scale, which grows as the scale shrinks. At scale 1 (11x the
    standard 1/sqrt(128)) the reference gradients reach |dQ| ~ 54, |dK| ~ 46, so they take
    the bound relative to their magnitude; at 0.02 the fixed bound."""
    test_fwd_bwd_parity((1, 8, 2, 512, 128, 4, "sparse", True, "normal"), scale=scale,
                        grad_scale_aware=scale > 0.1)


@pytest.mark.parametrize("case", [(1, 10, 2, 512, 128, 4, "sparse", True, "normal"),
                                  (1, 8, 2, 4096, 64, 8, "sparse", True, "zipf")],
                         ids=["G5", "zipf-split-lists"])
def test_deterministic_reruns(case):
    """Reruns give bit-identical outputs, also when the kernels take their work items in a
    permuted order (no atomics anywhere: every output element has one producer, the dg
    partials and the split key blocks' dK / dV partials are summed in a fixed order)."""
    _, a, *_ = _run(case)
    _, b, *_ = _run(case)
    try:
        sas.debug_workgroup_order(12345)
        _, c, *_ = _run(case)
        sas.debug_workgroup_order(7)
        _, d, *_ = _run(case)
    finally:
        sas.debug_workgroup_order(0)
    for k in ("idx", "cnt", "O", "lse", "dQ", "dK", "dV", "dg"):
        assert torch.equal(a[k], b[k]), k
        assert torch.equal(a[k], c[k]), ("permuted order", k)
        assert torch.equal(a[k], d[k]), ("permuted order", k)


def test_kernel_timing_records_each_launch():
    """The opt-in event timing sees every kernel of a training step, once per launch."""
    case = (1, 8, 2, 512, 128, 4, "sparse", True, "normal")
    sas.profile_enable(True)
    try:
        sas.profile_collect()
        _run(case)
        prof = sas.profile_collect()
    finally:
        sas.profile_enable(False)
    for name in ("select", "fwd", "inv_count", "inv_scan", "inv_fill", "dq", "dg_reduce", "dkv"):
        assert name in prof, (name, prof)
        launches, ms = prof[name]
        assert launches == 1 and ms > 0.0, (name, prof[name])
    assert sas.profile_collect() == {}


def test_kernel_timing_one_kernel():
    """With the one-kernel filter only that kernel's launches are recorded."""
    case = (1, 8, 2, 512, 128, 4, "sparse", True, "normal")
    sas.profile_enable(True)
    sas.profile_only("dkv")
    try:
        sas.profile_collect()
        _run(case)
        prof = sas.profile_collect()
    finally:
        sas.profile_only(None)
        sas.profile_enable(False)
    assert list(prof) == ["dkv"] and prof["dkv"][0] == 1 and prof["dkv"][1] > 0.0, prof


def _full_size(B, Hq, Hkv, n, d, topk, scores, nsample_j=6, nsample_m=3, backward=True, most_used=False):
    log(f"full size B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} K={topk} scores={scores}")
    P = Prefill(B, Hq, Hkv, n, d, seed=0, scores=scores, backward=backward)
    t = P.device()
    NB, G = P.NB, Hq // Hkv
    idx, cnt, _, logg = sas.sas_topk_select(t["s"], topk, cols=NB)
    O, lse = sas.sas_attn_fwd(t["Q"], t["K"], t["V"], idx, cnt, logg, P.scale)
    if backward:
        dQ, dK, dV, dg = sas.sas_attn_bwd(t["Q"], t["K"], t["V"], O, t["dO"], lse, idx, cnt, logg, P.scale)
    torch.cuda.synchronize()
    log("  GPU done; oracle selection")
    idx_r, cnt_r, _, logg_r = oracle.select_prefill(P.s, topk)
    assert np.array_equal(host(idx), idx_r) and np.array_equal(host(cnt), cnt_r)
    Q, K, V = P.f32("q"), P.f32("k"), P.f32("v")
    dO = P.f32("do") if backward else None
    g = np.random.default_rng(1)
    js = sorted(set([0, 1, NB - 1] + list(g.integers(2, NB - 1, nsample_j))))
    Oh = host(O)
    lseh = host(lse)
    if backward:
        dQh, dgh = host(dQ), host(dg)
    for j in js:
        h = int(g.integers(0, Hkv))
        rows = slice(j * 64, (j + 1) * 64)
        o_r, l_r = oracle.fwd_query_block(Q, K, V, 0, h, j, idx_r[0, h, j], cnt_r[0, h, j], logg_r[0, h, j], P.scale)
        assert_close(f"O[j={j},h={h}]", Oh[0, h * G:(h + 1) * G, rows], o_r)
        assert_close(f"LSE[j={j},h={h}]", lseh[0, h * G:(h + 1) * G, rows], l_r)
        if backward:
            dq_r, _, _, _, dg_r = oracle.bwd_query_block(Q, K, V, dO, 0, h, j, idx_r[0, h, j], cnt_r[0, h, j],
                                                         logg_r[0, h, j], P.scale)
            assert_close(f"dQ[j={j},h={h}]", dQh[0, h * G:(h + 1) * G, rows], dq_r)
            if cnt_r[0, h, j] > 0:
                assert_close(f"dg[j={j},h={h}]", dgh[0, h, j, :cnt_r[0, h, j]], dg_r, scale_aware=True)
    if not backward:
        return
    dKh, dVh = host(dK), host(dV)
    picks = [(0, int(g.integers(0, Hkv)))] + [(int(mm), int(g.integers(0, Hkv))) for mm in g.integers(1, NB, nsample_m)]
    if most_used:
        # for one head, also the key block with the most users: with skewed scores its
        # list is cut into several key-major workgroups whose partials are summed
        hm = int(g.integers(0, Hkv))
        uses = np.bincount(np.concatenate([idx_r[0, hm, j, :cnt_r[0, hm, j]] for j in range(NB)]).astype(np.int64),
                           minlength=NB)
        picks.append((int(np.argmax(uses)), hm))
    for m, h in picks:
        users = [j for j in range(m + 1, NB) if m in idx_r[0, h, j, :cnt_r[0, h, j]]]
        dk_r = np.zeros((64, d)); dv_r = np.zeros((64, d))
        for j in [m] + users:
            _, keys, dks, dvs, _ = oracle.bwd_query_block(Q, K, V, dO, 0, h, j, idx_r[0, h, j], cnt_r[0, h, j],
                                                          logg_r[0, h, j], P.scale)
            sel = (keys >= m * 64) & (keys < (m + 1) * 64)
            dk_r[keys[sel] - m * 64] += dks[sel]
            dv_r[keys[sel] - m * 64] += dvs[sel]
        log(f"  key block m={m} h={h}: {len(users)} selecting query blocks")
        assert_close(f"dK[m={m},h={h}]", dKh[0, h, m * 64:(m + 1) * 64], dk_r)
        assert_close(f"dV[m={m},h={h}]", dVh[0, h, m * 64:(m + 1) * 64], dv_r)
    # invariants over every element: sum_i dK_i = 0, sum_i dV_i = sum of the group's dO rows
    sk = dK.double().sum(dim=2).abs()
    sa = dK.double().abs().sum(dim=2)
    assert bool((sk <= 1e-2 * sa).all()), float((sk / sa).max())
    sv = host(dV.double().sum(dim=2))
    sdo = dO.reshape(B, Hkv, G, n, d).sum(axis=(2, 3))
    # a sum over n * G rows (magnitude ~sqrt(n G), hundreds here): relative bound
    assert_close("sum dV", sv, sdo, scale_aware=True)


def test_full_size_qwen3_4b_train():
    _full_size(1, 32, 8, 32768, 128, 32, "normal")


def test_full_size_qwen3_14b_k32():
    _full_size(1, 40, 8, 32768, 128, 32, "zipf", nsample_j=4, nsample_m=2)


def test_full_size_qwen3_14b_k16():
    _full_size(1, 40, 8, 32768, 128, 16, "zipf", nsample_j=4, nsample_m=2, most_used=True)


def test_full_size_qwen3_14b_k64():
    _full_size(1, 40, 8, 32768, 128, 64, "zipf", nsample_j=4, nsample_m=2, most_used=True)


LONG_LIST_CASES = [
    # selection rows longer than the 64 entries a wave holds at once: the kernels reload
    # their lane-held window of the list (query-major passes) and walk inverse lists of
    # more than 64 query blocks (key-major pass)
    (1, 2, 1, 8320, 64, 0, "full", True, "normal"),        # full scope, 130 blocks: rows up to 129 entries
    (1, 2, 1, 8192, 128, 96, "sparse", True, "normal"),    # sparse scope, K = 96
    (1, 4, 1, 8192, 64, 80, "sparse", True, "zipf"),       # K = 80, G = 4, popular blocks split key-major lists
]


@pytest.mark.parametrize("case", LONG_LIST_CASES, ids=[f"B{c[0]}H{c[1]}-{c[2]}n{c[3]}d{c[4]}K{c[5]}{c[6]}"
                                                        for c in LONG_LIST_CASES])
def test_fwd_bwd_long_lists(case):
    """Every output against the oracle, element by element, with lists of more than 64
    blocks (the longest list of each case is asserted to exceed 64)."""
    B, Hq, Hkv, n, d, topk, scope, gated, scores = case
    NB = n // 64
    longest = NB - 1 if scope == "full" else min(topk, NB - 1)
    assert longest > 64
    test_fwd_bwd_parity(case)


def test_key_major_split_lists():
    """Zipf scores over 128 query blocks: the top-ranked key blocks are selected by nearly
    every later query block, so the key-major pass cuts their lists into several
    workgroups and sums the partial dK / dV. The most-used block is checked against the
    oracle with sampled others, plus the gradient invariants on every element."""
    B, Hq, Hkv, n, d, topk = 1, 10, 2, 8192, 128, 8
    P = Prefill(B, Hq, Hkv, n, d, seed=0, scores="zipf")
    idx_r, cnt_r, _, _ = oracle.select_prefill(P.s, topk)
    assert _key_major_splits(idx_r, cnt_r, Hq // Hkv)
    _full_size(B, Hq, Hkv, n, d, topk, "zipf", nsample_j=2, nsample_m=2, most_used=True)


def test_full_size_long_prefill_fwd():
    _full_size(1, 32, 8, 131072, 128, 64, "planted", nsample_j=4, backward=False)


OUT_CASES = [
    (1, 8, 2, 1024, 128, 4, "sparse", True, "normal"),
    (2, 8, 2, 512, 64, 3, "sparse", True, "normal"),
    (1, 10, 2, 768, 128, 6, "sparse", True, "zipf"),
    (1, 4, 1, 512, 128, 0, "full", True, "normal"),
]


@pytest.mark.parametrize("case", OUT_CASES, ids=[f"B{c[0]}H{c[1]}-{c[2]}n{c[3]}d{c[4]}K{c[5]}{c[6]}" for c in OUT_CASES])
def test_fwd_bwd_gate_outside(case):
    """The gate after the softmax (the alternative of the explainer's choice 1) against
    the oracle: O, LSE of the ungated logits, dQ, dK, dV and dg = sum p dO.v. Some
    scores are -inf, so kept blocks with gate 0 still count in the normaliser."""
    log(f"fwd/bwd gate outside {case}")
    B, Hq, Hkv, n, d, topk, scope, _, scores = case
    P = Prefill(B, Hq, Hkv, n, d, seed=5, scores=scores)
    P.s[..., ::5] = -np.inf
    t = P.device()
    NB = P.NB
    kcap = NB - 1 if scope == "full" else topk
    idx, cnt, _, logg = sas.sas_topk_select(t["s"], topk, scope=scope, kcap=kcap, cols=NB)
    O, lse = sas.sas_attn_fwd(t["Q"], t["K"], t["V"], idx, cnt, logg, P.scale, placement="outside")
    dQ, dK, dV, dg = sas.sas_attn_bwd(t["Q"], t["K"], t["V"], O, t["dO"], lse, idx, cnt, logg, P.scale,
                                      placement="outside")
    torch.cuda.synchronize()
    idx_r, cnt_r, _, logg_r = oracle.select_prefill(P.s, topk, full_scope=scope == "full", kcap=kcap)
    assert np.array_equal(host(idx), idx_r) and np.array_equal(host(cnt), cnt_r)
    assert np.isneginf(logg_r).any()
    Q, K, V, dO = P.f32("q"), P.f32("k"), P.f32("v"), P.f32("do")
    O_r, lse_r = oracle.attn_fwd(Q, K, V, idx_r, cnt_r, logg_r, P.scale, placement="outside")
    assert_close("O", host(O), O_r)
    assert_close("LSE", host(lse), lse_r)
    dQ_r, dK_r, dV_r, dg_r = oracle.attn_bwd(Q, K, V, dO, idx_r, cnt_r, logg_r, P.scale, placement="outside")
    assert_close("dQ", host(dQ), dQ_r)
    assert_close("dK", host(dK), dK_r)
    assert_close("dV", host(dV), dV_r)
    assert_close("dg", host(dg), dg_r, scale_aware=True)

"""GPU parity of sas_gates_bwd (gradient of the scores through the gate softmax) against
the oracle's gates_bwd.

Inputs: seeded scores (normal, zipf, integer ties with -0, -inf and NaN) and a seeded
N(0,1) upstream gradient dg. Score entries that no row may read are NaN, and the output
buffer starts as NaN, so a read past the valid history or an unwritten entry shows up.
The kernel recomputes g in fp32 from s and the LSE; the oracle works in fp64, hence the
tolerance of 1e-5 relative to the largest |ds| (fp32 rounding of exp and of a sum of up
to 8192 products). The chain test runs selection, forward, backward and this kernel on
the same device tensors and compares with the oracle's chain at the attention tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from learned_context_ranking_amd import sas, synth
from gpu_util import Prefill, assert_close, dev, host, log

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _close(name, got, ref):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    bound = TOL * max(1e-3, float(np.abs(ref).max()) if ref.size else 0.0)
    log(f"  {name}: max|d|={err:.3e} (bound {bound:.3e})")
    assert err <= bound, (name, err, bound)


def _poison_prefill(s):
    s = s.copy()
    NB = s.shape[2]
    s[..., np.triu(np.ones((NB, s.shape[3]), dtype=bool), 0)[:NB]] = np.nan
    return s


def _prefill_case(s, topk, scope="sparse", seed=0):
    B, H, NB, ld = s.shape
    kcap = max(NB - 1, 1) if scope == "full" else min(topk, ld)
    sd = dev(_poison_prefill(s))
    idx, cnt, lse, _ = sas.sas_topk_select(sd, topk, scope=scope, kcap=kcap, cols=NB)
    dg = synth.normal_f32((B, H, NB, kcap), seed, synth.TID_DG)
    out = torch.full_like(sd, float("nan"))
    ds = sas.sas_gates_bwd(sd, lse, idx, cnt, dev(dg), cols=NB, out=out)
    torch.cuda.synchronize()
    idx_r, cnt_r, _, _ = oracle.select_prefill(s, topk, full_scope=scope == "full", kcap=kcap)
    assert np.array_equal(host(idx), idx_r) and np.array_equal(host(cnt), cnt_r)
    ds_r = oracle.gates_bwd_prefill(s, idx_r, cnt_r, dg)
    got = host(ds)
    _close(f"ds NB={NB} K={topk} {scope}", got, ds_r)
    # entries past each row's history are exactly zero
    assert np.all(got[..., np.triu(np.ones((NB, ld), dtype=bool), 0)[:NB]] == 0.0)
    return got, ds_r


@pytest.mark.parametrize("NB,topk", [(16, 4), (100, 7), (129, 32), (512, 32), (300, 0), (70, 200)])
def test_gates_bwd_prefill(NB, topk):
    log(f"gates_bwd prefill NB={NB} K={topk}")
    s = synth.scores_normal((2, 3, NB, NB), seed=NB)
    got, _ = _prefill_case(s, topk, seed=NB)
    # the gate softmax Jacobian has g-weighted rows summing to zero: sum_m ds_m = 0
    assert np.abs(got.sum(axis=-1)).max() < 1e-5


def test_gates_bwd_full_scope_and_zipf():
    _prefill_case(synth.scores_normal((1, 2, 70, 70), seed=5), 0, scope="full")
    _prefill_case(synth.scores_zipf(1, 2, 256, 0), 32, seed=3)


def test_gates_bwd_ties_signed_zero_nan_inf():
    g = np.random.default_rng(3)
    NB = 200
    s = g.integers(-2, 3, size=(1, 2, NB, NB)).astype(np.float32)
    s[0, 0, :, ::7] = -0.0
    s[0, 1, :, ::11] = -np.inf
    s[0, 1, :, 5::13] = np.nan
    s[0, 0, 150, :150] = -np.inf        # a row with history but no finite score
    got, _ = _prefill_case(s, 16)
    assert np.all(got[0, 0, 150] == 0.0)
    # NaN and -inf scores have gate 0, hence ds = 0
    bad = ~np.isfinite(s)
    assert np.all(got[bad & ~np.triu(np.ones((NB, NB), dtype=bool), 0)[None, None]] == 0.0)


@pytest.mark.parametrize("cols", [1, 63, 64, 65, 1024, 4000, 8192])
def test_gates_bwd_decode_rows(cols):
    log(f"gates_bwd decode cols={cols}")
    B, H = 5, 3
    g = np.random.default_rng(cols)
    s = g.standard_normal((B, H, 1, cols)).astype(np.float32)
    valid = np.array([cols, 0, cols // 2, min(cols, 3), max(cols - 1, 0)], np.int32)
    sp = s.copy()
    for b in range(B):
        sp[b, :, :, valid[b]:] = np.nan
    topk = 16
    kcap = min(topk, cols)
    sd, rv = dev(sp), dev(valid)
    idx, cnt, lse, _ = sas.sas_topk_select(sd, topk, mode="decode", row_valid=rv, kcap=kcap)
    dg = synth.normal_f32((B, H, 1, kcap), cols, synth.TID_DG)
    out = torch.full_like(sd, float("nan"))
    ds = sas.sas_gates_bwd(sd, lse, idx, cnt, dev(dg), mode="decode", row_valid=rv, out=out)
    torch.cuda.synchronize()
    idx_r, cnt_r, _, _ = oracle.select(s.reshape(B * H, cols), np.repeat(valid, H), topk, kcap=kcap)
    ds_r = oracle.gates_bwd(s.reshape(B * H, cols), np.repeat(valid, H), idx_r, cnt_r, dg.reshape(B * H, kcap))
    _close(f"ds decode cols={cols}", host(ds).reshape(B * H, cols), ds_r)


def test_gates_bwd_score_gradient_chain():
    """select -> fwd -> bwd -> gates_bwd on device against the oracle's chain (dg from the
    oracle's backward), at the attention tolerance since dg carries bf16 rounding."""
    case = (1, 8, 2, 1024, 128, 8)
    B, Hq, Hkv, n, d, topk = case
    log(f"score-gradient chain {case}")
    P = Prefill(B, Hq, Hkv, n, d, seed=2, scores="normal")
    t = P.device()
    NB = P.NB
    idx, cnt, lse_s, logg = sas.sas_topk_select(t["s"], topk, cols=NB)
    O, lse = sas.sas_attn_fwd(t["Q"], t["K"], t["V"], idx, cnt, logg, P.scale)
    _, _, _, dg = sas.sas_attn_bwd(t["Q"], t["K"], t["V"], O, t["dO"], lse, idx, cnt, logg, P.scale)
    ds = sas.sas_gates_bwd(t["s"], lse_s, idx, cnt, dg.reshape(idx.shape), cols=NB)
    torch.cuda.synchronize()
    idx_r, cnt_r, _, logg_r = oracle.select_prefill(P.s, topk)
    Q, K, V, dO = P.f32("q"), P.f32("k"), P.f32("v"), P.f32("do")
    _, _, _, dg_r = oracle.attn_bwd(Q, K, V, dO, idx_r, cnt_r, logg_r, P.scale)
    ds_r = oracle.gates_bwd_prefill(P.s, idx_r, cnt_r, dg_r)
    # ds = g (dg - c) carries dg's magnitude and rounding, hence dg's scale-aware bound
    assert_close("ds (chain)", host(ds), ds_r, scale_aware=True)


def test_gates_bwd_full_size_train_scores():
    """Training-step selection (8 KV heads x 512 query blocks, K = 32) with a N(0,1)
    upstream dg: every row against the oracle."""
    log("gates_bwd full size: 8 x 512 x 512, K=32")
    s = synth.scores_normal((1, 8, 512, 512), seed=0)
    _prefill_case(s, 32, seed=11)


@pytest.mark.parametrize("gate", ["softmax_selected", "sigmoid", "exp"])
def test_gates_bwd_gate_variants(gate):
    """ds under each gate activation against the oracle (prefill rows with NaN-poisoned
    invalid entries, -inf scores, a budget above the history)."""
    log(f"gates_bwd gate={gate}")
    NB = 200
    s = synth.scores_normal((1, 3, NB, NB), seed=23)
    s[0, 2, :, ::13] = -np.inf
    for topk in (9, 250):
        kcap = min(topk, NB)
        sd = dev(_poison_prefill(s))
        idx, cnt, lse, _ = sas.sas_topk_select(sd, topk, kcap=kcap, cols=NB, gate=gate)
        dg = synth.normal_f32((1, 3, NB, kcap), topk, synth.TID_DG)
        out = torch.full_like(sd, float("nan"))
        ds = sas.sas_gates_bwd(sd, lse if gate == "softmax_selected" else None, idx, cnt, dev(dg), cols=NB, out=out,
                               gate=gate)
        torch.cuda.synchronize()
        idx_r, cnt_r, _, _ = oracle.select_prefill(s, topk, kcap=kcap, gate=gate)
        assert np.array_equal(host(idx), idx_r)
        ds_r = oracle.gates_bwd_prefill(s, idx_r, cnt_r, dg, gate=gate)
        _close(f"ds gate={gate} K={topk}", host(ds), ds_r)


def test_gates_bwd_variant_score_gradient_chain():
    """The sigmoid-gated step end to end on device: select -> fwd -> bwd -> gates_bwd."""
    B, Hq, Hkv, n, d, topk = 1, 8, 2, 1024, 128, 8
    P = Prefill(B, Hq, Hkv, n, d, seed=4, scores="normal")
    t = P.device()
    idx, cnt, _, logg = sas.sas_topk_select(t["s"], topk, cols=P.NB, gate="sigmoid")
    O, lse = sas.sas_attn_fwd(t["Q"], t["K"], t["V"], idx, cnt, logg, P.scale)
    _, _, _, dg = sas.sas_attn_bwd(t["Q"], t["K"], t["V"], O, t["dO"], lse, idx, cnt, logg, P.scale)
    ds = sas.sas_gates_bwd(t["s"], None, idx, cnt, dg.reshape(idx.shape), cols=P.NB, gate="sigmoid")
    torch.cuda.synchronize()
    idx_r, cnt_r, _, logg_r = oracle.select_prefill(P.s, topk, gate="sigmoid")
    assert np.array_equal(host(idx), idx_r)
    Q, K, V, dO = P.f32("q"), P.f32("k"), P.f32("v"), P.f32("do")
    _, _, _, dg_r = oracle.attn_bwd(Q, K, V, dO, idx_r, cnt_r, logg_r, P.scale)
    ds_r = oracle.gates_bwd_prefill(P.s, idx_r, cnt_r, dg_r, gate="sigmoid")
    assert_close("ds (sigmoid chain)", host(ds), ds_r, scale_aware=True)

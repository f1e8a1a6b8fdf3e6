"""The entry points recorded in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Each call only launches kernels on the caller's stream: no allocation, no memset and no
host synchronisation inside the library, so a whole training step (select, forward,
backward) or decode step (select, decode, chunk merge; or the decode with its selection) can
be captured once. The kernels are deterministic, so every replay must reproduce the eager
results bit for bit; the outputs are overwritten with garbage before each replay, and
unrelated eager work and synchronisations run between replays.
"""
import math

import numpy as np
import pytest
import torch

from learned_context_ranking_amd import sas, synth
from gpu_util import Prefill, dev, dev_bf16, log

pytestmark = pytest.mark.gpu


def _poison(out):
    for t in out.values():
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


def _replays(graph, out, ref, n=3):
    for r in range(n):
        _poison(out)
        x = torch.randn(512, 512, device="cuda")
        (x @ x).sum().item()   # eager work and a host synchronisation between replays
        graph.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(out[k], ref[k]), f"replay {r}: {k} differs from the eager result"
        log(f"  replay {r}: {len(ref)} outputs equal to the eager run")


def test_train_step_graph_replay():
    B, Hq, Hkv, n, d, topk = 1, 8, 2, 4096, 128, 8
    log(f"graph: training step B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} K={topk} (zipf: split key-major lists)")
    P = Prefill(B, Hq, Hkv, n, d, seed=4, scores="zipf")
    t = P.device()
    NB = n // 64
    ws = sas.bwd_workspace(B, Hq, Hkv, n, d, topk, t["Q"].device)

    def step():
        idx, cnt, _, logg = sas.sas_topk_select(t["s"], topk, kcap=topk, cols=NB)
        O, lse = sas.sas_attn_fwd(t["Q"], t["K"], t["V"], idx, cnt, logg, P.scale)
        dQ, dK, dV, dg = sas.sas_attn_bwd(t["Q"], t["K"], t["V"], O, t["dO"], lse, idx, cnt, logg, P.scale, ws=ws)
        return dict(idx=idx, cnt=cnt, logg=logg, O=O, lse=lse, dQ=dQ, dK=dK, dV=dV, dg=dg)

    ref = {k: v.clone() for k, v in step().items()}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    _replays(g, out, ref)


@pytest.mark.parametrize("B,Hkv,Lmax", [(2, 2, 4096), (64, 8, 1024)], ids=["merged-chunks", "one-chunk"])
def test_decode_step_graph_replay(B, Hkv, Lmax):
    Hq, d, topk = 4 * Hkv, 128, 16
    log(f"graph: decode step B={B} Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} K={topk}")
    q = dev_bf16(synth.normal_bf16((B, Hq, 1, d), 2, synth.TID_QDEC)[:, :, 0])
    Kc = dev_bf16(synth.normal_bf16((B, Hkv, Lmax, d), 2, synth.TID_K))
    Vc = dev_bf16(synth.normal_bf16((B, Hkv, Lmax, d), 2, synth.TID_V))
    C = Lmax // 64
    s = dev(synth.scores_normal((B, Hkv, 1, C), 2))
    kv_len_h = np.linspace(100, Lmax, B).astype(np.int32)
    kv_len = dev(kv_len_h)
    row_valid = dev(((kv_len_h - 1) // 64).astype(np.int32))
    scale = 1.0 / math.sqrt(d)
    ws = sas.decode_workspace(B, Hq, Hkv, d, topk, q.device)

    def step():
        idx, cnt, _, logg = sas.sas_topk_select(s, topk, mode="decode", row_valid=row_valid, kcap=topk)
        o = sas.sas_decode(q, Kc, Vc, kv_len, idx, cnt, scale, logg=logg, ws=ws)
        return dict(idx=idx, cnt=cnt, o=o)

    ref = {k: v.clone() for k, v in step().items()}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    _replays(g, out, ref)


@pytest.mark.parametrize("B,Hkv,Lmax", [(2, 2, 4096), (64, 8, 1024)], ids=["merged-chunks", "one-chunk"])
def test_decode_topk_graph_replay(B, Hkv, Lmax):
    """The decode with its selection in the launch, captured and replayed: kept blocks
    (idx_out / cnt_out) and output."""
    Hq, d, topk = 4 * Hkv, 128, 16
    log(f"graph: decode_topk B={B} Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} K={topk}")
    q = dev_bf16(synth.normal_bf16((B, Hq, 1, d), 3, synth.TID_QDEC)[:, :, 0])
    Kc = dev_bf16(synth.normal_bf16((B, Hkv, Lmax, d), 3, synth.TID_K))
    Vc = dev_bf16(synth.normal_bf16((B, Hkv, Lmax, d), 3, synth.TID_V))
    s = dev(synth.scores_normal((B, Hkv, 1, Lmax // 64), 3))
    kv_len = dev(np.linspace(100, Lmax, B).astype(np.int32))
    scale = 1.0 / math.sqrt(d)
    ws = sas.decode_workspace(B, Hq, Hkv, d, topk, q.device)

    def step():
        o, idx, cnt = sas.sas_decode_topk(q, Kc, Vc, kv_len, s, topk, scale, ws=ws, want_idx=True)
        return dict(idx=idx, cnt=cnt, o=o)

    ref = {k: v.clone() for k, v in step().items()}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    _replays(g, out, ref)


def test_decode_long_graph_replay():
    """The two-launch long-context decode (candidates in the workspace, then the decode
    ranking them), captured and replayed."""
    B, Hq, Hkv, d, Lmax, topk = 2, 8, 2, 128, 65536, 16
    log(f"graph: decode_long B={B} Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} K={topk}")
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    Kc = torch.randn((B, Hkv, Lmax, d), generator=g, device="cuda").to(torch.bfloat16)
    Vc = torch.randn((B, Hkv, Lmax, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    kv_len = dev(np.array([Lmax, 20000], np.int32))
    kbar = sas.sas_pool_keys(Kc, kv_len)
    ws = sas.decode_long_workspace(B, Hq, Hkv, d, Lmax // 64, topk, q.device)
    scale = 1.0 / math.sqrt(d)

    def step():
        o, idx, cnt = sas.sas_decode_long(q, kbar, Kc, Vc, kv_len, topk, scale, ws=ws, want_idx=True)
        return dict(idx=idx, cnt=cnt, o=o)

    ref = {k: v.clone() for k, v in step().items()}
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        out = step()
    _replays(gr, out, ref)

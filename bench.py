#!/usr/bin/env python3
"""Benchmark of the SAS log-gated block-sparse attention hot path on one MI355X.

A step is one pass of the training hot path over the Qwen3-4B-shaped single-layer
workload (batch 1, 32 query / 8 KV heads, head_dim 128, n = 32,768, block 64, Top-K 32,
bf16 Q/K/V/dO ~ N(0,1), fp32 scores ~ N(0,1)): gate + Top-K selection, gated forward,
backward with dQ, dK, dV and dg, and the score gradient ds through the gate softmax.
Inputs are resident in HBM before timing starts.

value = algorithmic FLOPs / step time, counting only attended (query, key) pairs:
4*d per pair forward (q.k, p.v) and 8*d backward (dO.v, p^T dO, dS k, dS^T q); the
backward's recomputation of q.k is not counted. The roofline object covers the kernel
with the longest launch (the key-major dK/dV pass), timed with the library's per-kernel
HIP events over the timed region; its traffic comes from profiles/traffic_<kernel>.txt
while the kernel's sources match the digest taken with the counters. The decode workload
(64 sequences, 32,768 cached tokens, 16 blocks + the current block per KV head) is
reported alongside as HBM GB/s of the decode kernel, with L2 / Infinity Cache evicted by
a 1 GiB read before each launch. The long-context decode object times one decode step's
selection (block scores over the pooled-key cache + Top-K) against its sparse attention
at 32K-512K cached tokens. The sweep object times the other prefill configurations (the
128K-token long prefill forward and the Qwen3-14B-shaped budgets 16 / 32 / 64) by the same
FLOP counting.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def calibration_copy(torch, nbytes=256 << 20):
    """A plain copy of a known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy: {nbytes} bytes read, {nbytes} bytes written")


def stats(samples) -> dict:
    """mean / median / p10 / p90 (ms) of a list of per-launch or per-step times."""
    a = np.asarray(samples, np.float64)
    return {"mean": round(float(a.mean()), 5), "median": round(float(np.median(a)), 5),
            "p10": round(float(np.percentile(a, 10)), 5), "p90": round(float(np.percentile(a, 90)), 5),
            "n": int(a.size)}


def select_bytes(NB: int, rows_per_head: int, H: int, kcap: int) -> int:
    """Algorithmic bytes of one prefill selection launch: the valid scores read (row j has
    j of them) and idx, logg (kcap each), cnt and lse written per row."""
    valid = NB * (NB - 1) // 2 * H
    return 4 * valid + rows_per_head * H * (8 * kcap + 8)


def measure_peaks(torch, reps=5):
    """Measured ceilings on this machine: the bf16 MFMA rate of an MFMA-loop microkernel (with
    the shader clock under that load, from the in-kernel cycle and 100 MHz counters) and
    the rate of a streaming read of 2 GiB (L2 / Infinity Cache hold a small part of it)."""
    from learned_context_ranking_amd import sas
    dev = torch.device("cuda", 0)
    wgs, iters = 2048, 2000
    clocks = torch.zeros(2 * wgs, dtype=torch.int64, device=dev)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    flop = wgs * 4 * iters * 8 * 32768.0
    sas.measure_mfma(wgs, iters, clocks, sink)
    mf, rd = [], []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        sas.measure_mfma(wgs, iters, clocks, sink)
        b.record(stream)
        b.synchronize()
        mf.append(a.elapsed_time(b))
    c = clocks.reshape(-1, 2).double().cpu().numpy()
    sclk_mhz = float(np.median(c[:, 0] / np.maximum(c[:, 1], 1)) * 100.0)
    buf = torch.ones((1 << 29,), dtype=torch.float32, device=dev)   # 2 GiB
    sas.measure_read(buf, sink)
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        sas.measure_read(buf, sink)
        b.record(stream)
        b.synchronize()
        rd.append(a.elapsed_time(b))
    del buf
    tf = flop / (float(np.median(mf)) * 1e-3) / 1e12
    gbs = (1 << 31) / (float(np.median(rd)) * 1e-3) / 1e9
    return {"mfma_bf16_tflops": round(tf, 1), "sclk_mhz_under_mfma_load": round(sclk_mhz, 1),
            "stream_read_gbs": round(gbs, 1),
            "method": "sas_measure_mfma: 2048 workgroups x 4 waves x 2000 rounds of 8 independent bf16 "
                      "32x32x16 MFMAs, median of 5 launches; clock = s_memtime cycles / s_memrealtime "
                      "ticks x 100 MHz over wave 0 of each workgroup; sas_measure_read: 2 GiB streamed "
                      "with 16-byte loads, median of 5"}


def pair_count(cnt: np.ndarray, G: int, block: int = 64) -> int:
    """Attended (query row, key) pairs: causal current block plus cnt_j full history
    blocks for every query block, times the G query heads of each KV head."""
    per_block = block * (block + 1) // 2 + cnt.astype(np.int64) * block * block
    return int(per_block.sum()) * G


def bf16_device(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def train_inputs(w, torch):
    from learned_context_ranking_amd import synth
    q = synth.normal_bf16((w.B, w.Hq, w.n, w.d), w.seed, synth.TID_Q)
    k = synth.normal_bf16((w.B, w.Hkv, w.n, w.d), w.seed, synth.TID_K)
    v = synth.normal_bf16((w.B, w.Hkv, w.n, w.d), w.seed, synth.TID_V)
    do = synth.normal_bf16((w.B, w.Hq, w.n, w.d), w.seed, synth.TID_DO)
    s = synth.prefill_scores(w)
    host = dict(q=q, k=k, v=v, do=do, s=s)
    dev = dict(Q=bf16_device(q, torch), K=bf16_device(k, torch), V=bf16_device(v, torch),
               dO=bf16_device(do, torch), s=torch.from_numpy(s).cuda())
    return host, dev


TIMED_KERNEL = "dkv"   # the training step's dominant kernel, timed live in the timed region


def run_train(w, steps, warmup, torch, kernel_timing=True):
    from learned_context_ranking_amd import sas
    log(f"[bench] generating {w.name} inputs")
    host, t = train_inputs(w, torch)
    scale = 1.0 / math.sqrt(w.d)
    NB = w.NB
    dev = t["Q"].device
    idx = torch.empty((w.B, w.Hkv, NB, w.topk), dtype=torch.int32, device=dev)
    # outputs and workspace allocated once, outside the timed region
    O = torch.empty_like(t["Q"])
    lse = torch.empty((w.B, w.Hq, w.n), dtype=torch.float32, device=dev)
    dQ = torch.empty(t["Q"].shape, dtype=torch.float32, device=dev)
    dK = torch.empty(t["K"].shape, dtype=torch.float32, device=dev)
    dV = torch.empty(t["V"].shape, dtype=torch.float32, device=dev)
    dg = torch.empty((w.B, w.Hkv, NB, w.topk), dtype=torch.float32, device=dev)
    ds = torch.empty_like(t["s"])
    ws = sas.bwd_workspace(w.B, w.Hq, w.Hkv, w.n, w.d, w.topk, dev)
    stream = torch.cuda.current_stream()
    ev = {k: [] for k in ("sel", "fwd", "bwd", "gates_bwd")}

    ev["step"] = []

    def step(record):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
        if record:
            marks[0].record(stream)
        idx_, cnt_, lse_s, logg_ = sas.sas_topk_select(t["s"], w.topk, kcap=w.topk, cols=NB)
        if record:
            marks[1].record(stream)
        sas.sas_attn_fwd(t["Q"], t["K"], t["V"], idx_, cnt_, logg_, scale, out=O, lse_out=lse)
        if record:
            marks[2].record(stream)
        sas.sas_attn_bwd(t["Q"], t["K"], t["V"], O, t["dO"], lse, idx_, cnt_, logg_, scale, ws=ws,
                         outs=(dQ, dK, dV, dg))
        if record:
            marks[3].record(stream)
        # gradient of the scores through the gate softmax
        sas.sas_gates_bwd(t["s"], lse_s, idx_, cnt_, dg, cols=NB, out=ds)
        if record:
            marks[4].record(stream)
            ev["sel"].append((marks[0], marks[1]))
            ev["fwd"].append((marks[1], marks[2]))
            ev["bwd"].append((marks[2], marks[3]))
            ev["gates_bwd"].append((marks[3], marks[4]))
            ev["step"].append((marks[0], marks[4]))
        return cnt_

    log(f"[bench] warmup {warmup}")
    for _ in range(warmup):
        cnt = step(False)
    torch.cuda.synchronize()
    cnt = step(False)
    torch.cuda.synchronize()
    cnt_h = cnt.cpu().numpy()
    pairs = pair_count(cnt_h, w.G)
    flop_fwd = 4.0 * w.d * pairs
    flop_bwd = 8.0 * w.d * pairs
    log(f"[bench] timing {steps} steps")
    torch.cuda.synchronize()
    sas.profile_collect()            # drop anything recorded before the timed region
    # Inside the timed region only the dominant kernel (the key-major pass) is bracketed by
    # HIP events on its launch stream (the roofline's live launch time); events around every
    # kernel would add ~0.1 ms to each step. The per-kernel breakdown comes from the same
    # steps run again with every kernel bracketed, after the timed region.
    sas.profile_enable(kernel_timing)
    sas.profile_only(TIMED_KERNEL)
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sas.profile_enable(False)
    sas.profile_only(None)
    timed_launches = sas.profile_collect_launches()
    ms_step = (t1 - t0) * 1e3 / steps
    ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    ev_stats = {k: stats([a.elapsed_time(b) for a, b in v]) for k, v in ev.items()}
    launches = []
    if kernel_timing:
        sas.profile_enable(True)
        for _ in range(steps):
            step(False)
        torch.cuda.synchronize()
        sas.profile_enable(False)
        launches = sas.profile_collect_launches()
    per_kernel = {}
    for name, t_ms in launches:
        per_kernel.setdefault(name, []).append(t_ms)
    timed = [t_ms for name, t_ms in timed_launches if name == TIMED_KERNEL]
    if timed:
        per_kernel[TIMED_KERNEL] = timed
    kern_ms = {k: float(np.mean(v)) for k, v in per_kernel.items()}
    kern_stats = {k: stats(v) for k, v in per_kernel.items()}
    # the same forward + backward with the gate placed after the softmax (the design
    # alternative the method is compared with), on the same selection
    idx_, cnt_, _, logg_ = sas.sas_topk_select(t["s"], w.topk, kcap=w.topk, cols=NB)
    outside = []
    for r in range(steps + 2):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        sas.sas_attn_fwd(t["Q"], t["K"], t["V"], idx_, cnt_, logg_, scale, out=O, lse_out=lse, placement="outside")
        sas.sas_attn_bwd(t["Q"], t["K"], t["V"], O, t["dO"], lse, idx_, cnt_, logg_, scale, ws=ws,
                         outs=(dQ, dK, dV, dg), placement="outside")
        b_.record(stream)
        if r >= 2:
            outside.append((a_, b_))
    torch.cuda.synchronize()
    ms["fwd_bwd_gate_outside"] = float(np.mean([a_.elapsed_time(b_) for a_, b_ in outside]))
    # score-gradient norm under the method's gate (softmax over the history) against the
    # kept-set normalisation of a binary Top-K mask ([SAS-ko] choice 3), same inputs
    gnorm = {}
    for gate in ("softmax", "softmax_selected"):
        idx_, cnt_, lse_s, logg_ = sas.sas_topk_select(t["s"], w.topk, kcap=w.topk, cols=NB, gate=gate)
        sas.sas_attn_fwd(t["Q"], t["K"], t["V"], idx_, cnt_, logg_, scale, out=O, lse_out=lse)
        sas.sas_attn_bwd(t["Q"], t["K"], t["V"], O, t["dO"], lse, idx_, cnt_, logg_, scale, ws=ws,
                         outs=(dQ, dK, dV, dg))
        sas.sas_gates_bwd(t["s"], lse_s, idx_, cnt_, dg, cols=NB, out=ds, gate=gate)
        gnorm[gate] = float(torch.linalg.vector_norm(ds.double()))
    gnorm["ratio"] = gnorm["softmax_selected"] / gnorm["softmax"]
    return dict(ms_step=ms_step, ms=ms, kern_ms=kern_ms, pairs=pairs, flop_fwd=flop_fwd,
                flop_bwd=flop_bwd, host=host, cnt=cnt_h, ev_stats=ev_stats, kern_stats=kern_stats,
                gate_grad_norm=gnorm)


def run_decode(steps, torch):
    """Decode workload: one new token per sequence over a 32,768-token cache."""
    from learned_context_ranking_amd import sas, synth
    w = synth.WORKLOADS["decode"]
    B, Hq, Hkv, d, L, K = w.B, w.Hq, w.Hkv, w.d, w.n, w.topk
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    log("[bench] generating decode caches on device (seeded)")
    Kc = torch.randn((B, Hkv, L, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    Vc = torch.randn((B, Hkv, L, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    C = L // 64
    s = torch.from_numpy(synth.scores_normal((B, Hkv, 1, C), w.seed)).to(dev)
    kv_len = torch.full((B,), L, dtype=torch.int32, device=dev)
    row_valid = ((kv_len - 1) // 64).to(torch.int32)
    idx, cnt, _, _ = sas.sas_topk_select(s, K, mode="decode", row_valid=row_valid, kcap=K)
    ws = sas.decode_workspace(B, Hq, Hkv, d, K, dev)
    o = torch.empty_like(q)
    # Evict the caches before each timed step by READING 1 GiB (> L2 + Infinity Cache).
    # A write flush (zero_) would leave ~256 MB of dirty lines whose write-back then
    # competes with the timed kernel's reads and halves its measured bandwidth.
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    scale = 1.0 / math.sqrt(d)
    for _ in range(3):
        sas.sas_decode(q, Kc, Vc, kv_len, idx, cnt, scale, ws=ws, out=o)
    torch.cuda.synchronize()
    times, sel_times = [], []
    for _ in range(steps):
        flush.sum()
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record(stream)
        sas.sas_topk_select(s, K, mode="decode", row_valid=row_valid, kcap=K)
        b.record(stream)
        sas.sas_decode(q, Kc, Vc, kv_len, idx, cnt, scale, ws=ws, out=o)
        c.record(stream)
        times.append((b, c))
        sel_times.append((a, b))
    torch.cuda.synchronize()
    dec_samples = [x.elapsed_time(y) for x, y in times]
    sel_samples = [x.elapsed_time(y) for x, y in sel_times]
    # Steady state of a serving loop: `steps` decode steps back to back on the stream (no
    # host sync, no flush between them), each over the selection of one of 4 score draws in
    # turn, so a step's 286 MB gather is not in the 256 MB Infinity Cache (the 3 steps
    # since the same selection was used read ~860 MB of other blocks). Events bracket each
    # step; dispatch of a step overlaps the previous one, as in a serving loop.
    sel_sets = []
    for r in range(4):
        s_r = torch.from_numpy(synth.scores_normal((B, Hkv, 1, C), w.seed + 101 + r)).to(dev)
        sel_sets.append(sas.sas_topk_select(s_r, K, mode="decode", row_valid=row_valid, kcap=K)[:2])
    o_ss = torch.empty_like(q)
    for i in range(8):
        sas.sas_decode(q, Kc, Vc, kv_len, sel_sets[i % 4][0], sel_sets[i % 4][1], scale, ws=ws, out=o_ss)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(steps):
        sas.sas_decode(q, Kc, Vc, kv_len, sel_sets[i % 4][0], sel_sets[i % 4][1], scale, ws=ws, out=o_ss)
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    ss_samples = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
    # The same steady state replayed from a HIP graph (the pages' decode measurements run
    # under CUDA graphs in their serving stack): GSTEPS steps over the 4 selections captured
    # once and replayed, with no host call, event or launch latency between the steps.
    GSTEPS = 20
    o_g = torch.empty_like(q)
    gstream = torch.cuda.Stream()
    gstream.wait_stream(stream)
    with torch.cuda.stream(gstream):
        for i in range(4):
            sas.sas_decode(q, Kc, Vc, kv_len, sel_sets[i][0], sel_sets[i][1], scale, ws=ws, out=o_g)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gstream):
        for i in range(GSTEPS):
            sas.sas_decode(q, Kc, Vc, kv_len, sel_sets[i % 4][0], sel_sets[i % 4][1], scale, ws=ws, out=o_g)
    graph.replay()
    torch.cuda.synchronize()
    last = (GSTEPS - 1) % 4
    sas.sas_decode(q, Kc, Vc, kv_len, sel_sets[last][0], sel_sets[last][1], scale, ws=ws, out=o_ss)
    torch.cuda.synchronize()
    assert torch.equal(o_g, o_ss), "graph-replayed decode differs from the eager decode"
    gtimes = []
    for _ in range(max(10, steps // GSTEPS)):
        a_, c_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        graph.replay()
        c_.record(stream)
        gtimes.append((a_, c_))
    torch.cuda.synchronize()
    graph_samples = [x.elapsed_time(y) / GSTEPS for x, y in gtimes]
    del graph
    # event-to-event time of a trivial kernel on the same stream (the dispatch floor that
    # every isolated, event-bracketed launch carries)
    tiny = torch.zeros(64, device=dev)
    tt = []
    for _ in range(50):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        tiny.add_(1.0)
        b_.record(stream)
        b_.synchronize()
        tt.append(a_.elapsed_time(b_))
    dispatch_ms = float(np.median(tt))
    ss_blocks = [int(c.sum().item()) + B * Hkv for _, c in sel_sets]
    ss_bytes = float(np.mean(ss_blocks)) * 64 * d * 2 * 2 + 2 * B * Hq * d * 2
    e2e_samples = [x[0].elapsed_time(y[1]) for x, y in zip(sel_times, times)]
    ms = float(np.median(dec_samples))
    ms_sel = float(np.median(sel_samples))
    # the same step over a paged cache: the sequences' blocks scattered over a pool of
    # 64-token pages in random order, read through a page table
    C = L // 64
    perm = torch.randperm(B * C, generator=torch.Generator().manual_seed(7))
    Kp = Kc.reshape(B, Hkv, C, 64, d).permute(0, 2, 1, 3, 4).reshape(B * C, Hkv, 64, d)[perm.to(dev)].contiguous()
    Vp = Vc.reshape(B, Hkv, C, 64, d).permute(0, 2, 1, 3, 4).reshape(B * C, Hkv, 64, d)[perm.to(dev)].contiguous()
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(B * C)
    page_table = inv.reshape(B, C).to(torch.int32).to(dev)
    op = torch.empty_like(q)
    for _ in range(3):
        sas.sas_decode_paged(q, Kp, Vp, page_table, kv_len, idx, cnt, scale, ws=ws, out=op)
    torch.cuda.synchronize()
    assert torch.equal(op, o), "paged decode differs from the contiguous decode"
    ptimes = []
    for _ in range(steps):
        flush.sum()
        a, c = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        a.record(stream)
        sas.sas_decode_paged(q, Kp, Vp, page_table, kv_len, idx, cnt, scale, ws=ws, out=op)
        c.record(stream)
        ptimes.append((a, c))
    torch.cuda.synchronize()
    paged_samples = [x.elapsed_time(y) for x, y in ptimes]
    ms_paged = float(np.median(paged_samples))
    # the paged step with its selection in the launch
    opf = torch.empty_like(q)
    sas.sas_decode_paged_topk(q, Kp, Vp, page_table, kv_len, s, K, scale, ws=ws, out=opf)
    torch.cuda.synchronize()
    assert torch.equal(opf, o), "paged fused decode differs from select + decode"
    pftimes = []
    for _ in range(steps):
        flush.sum()
        a, c = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        a.record(stream)
        sas.sas_decode_paged_topk(q, Kp, Vp, page_table, kv_len, s, K, scale, ws=ws, out=opf)
        c.record(stream)
        pftimes.append((a, c))
    torch.cuda.synchronize()
    paged_fused_samples = [x.elapsed_time(y) for x, y in pftimes]
    del Kp, Vp
    # the same step with the mass-threshold early stop (blocks in descending score order)
    order = torch.gather(s[:, :, 0, :], -1, idx.reshape(B, Hkv, -1).clamp(min=0).long()).contiguous()
    early = {}
    for tau in (0.0, 0.1):
        oe, used = sas.sas_decode_early_stop(q, Kc, Vc, kv_len, idx, cnt, order, scale, tau)
        torch.cuda.synchronize()
        et = []
        for _ in range(steps):
            flush.sum()
            a, c = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            a.record(stream)
            sas.sas_decode_early_stop(q, Kc, Vc, kv_len, idx, cnt, order, scale, tau, out=oe, used=used)
            c.record(stream)
            et.append((a, c))
        torch.cuda.synchronize()
        early[tau] = (float(np.median([x.elapsed_time(y) for x, y in et])), float(used.float().mean()))
    # the same step with the selection inside the decode launch (sas_decode_topk): one
    # isolated launch after the flush, and steps back to back over the 4 score draws
    of = torch.empty_like(q)
    sas.sas_decode_topk(q, Kc, Vc, kv_len, s, K, scale, ws=ws, out=of)
    torch.cuda.synchronize()
    assert torch.equal(of, o), "fused decode differs from select + decode"
    ftimes = []
    for _ in range(steps):
        flush.sum()
        a, c = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        a.record(stream)
        sas.sas_decode_topk(q, Kc, Vc, kv_len, s, K, scale, ws=ws, out=of)
        c.record(stream)
        ftimes.append((a, c))
    torch.cuda.synchronize()
    fused_samples = [x.elapsed_time(y) for x, y in ftimes]
    s_draws = [torch.from_numpy(synth.scores_normal((B, Hkv, 1, C), w.seed + 101 + r)).to(dev) for r in range(4)]
    fmarks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    fmarks[0].record(stream)
    for i in range(steps):
        sas.sas_decode_topk(q, Kc, Vc, kv_len, s_draws[i % 4], K, scale, ws=ws, out=of)
        fmarks[i + 1].record(stream)
    torch.cuda.synchronize()
    fss_samples = [fmarks[i].elapsed_time(fmarks[i + 1]) for i in range(steps)]
    cnt_h = cnt.cpu().numpy()
    # algorithmic bytes: the selected K/V blocks plus the current block, q and o
    blocks = int(cnt_h.sum()) + B * Hkv
    nbytes = blocks * 64 * d * 2 * 2 + 2 * B * Hq * d * 2
    # selection: the row's valid scores read, idx (kcap), cnt and lse written
    sel_bytes = B * Hkv * ((L - 1) // 64) * 4 + B * Hkv * (4 * K + 8)
    ms_e2e = float(np.median(e2e_samples))
    # fused: the decode bytes plus the scores each row's workgroup reads (no idx/cnt written)
    fused_bytes = nbytes + B * Hkv * ((L - 1) // 64) * 4
    return dict(ms=ms, ms_select=ms_sel, bytes=nbytes, gbs=nbytes / ms / 1e6, ms_paged=ms_paged,
                gbs_paged=nbytes / ms_paged / 1e6, early=early, stats=stats(dec_samples),
                sel_stats=stats(sel_samples), paged_stats=stats(paged_samples), sel_bytes=sel_bytes,
                sel_gbs=sel_bytes / ms_sel / 1e6, ms_e2e=ms_e2e, e2e_stats=stats(e2e_samples),
                ss_stats=stats(ss_samples), ss_bytes=ss_bytes, dispatch_ms=dispatch_ms,
                ss_gbs=ss_bytes / float(np.median(ss_samples)) / 1e6,
                graph_stats=stats(graph_samples), graph_gbs=ss_bytes / float(np.median(graph_samples)) / 1e6,
                graph_steps=GSTEPS,
                ms_fused=float(np.median(fused_samples)), fused_stats=stats(fused_samples), fused_bytes=fused_bytes,
                fss_stats=stats(fss_samples), fss_ms=float(np.median(fss_samples)),
                paged_fused_stats=stats(paged_fused_samples), ms_paged_fused=float(np.median(paged_fused_samples)),
                e2e_gbs=(nbytes + sel_bytes) / ms_e2e / 1e6,
                workload=f"decode: B={B} sequences, Hq={Hq}, Hkv={Hkv}, d={d}, kv_len={L}, block=64, "
                         f"K={K} blocks + current block, ungated (Algorithm 2)")


def run_long_decode(torch, reps=20):
    """Long-context decode selection: one decode step's block scoring + Top-K
    (sas_decode_select over the pooled-key cache) against its sparse attention
    (sas_decode) at 32K, 128K and 512K cached tokens, batch 1 and 8, 32 query / 8 KV heads,
    d = 128, K = 16. The caches are allocated once at 512K capacity; kv_len sets the
    context. Pooling is not timed: each block is pooled once, when it completes."""
    from learned_context_ranking_amd import sas
    dev = torch.device("cuda", 0)
    Bmax, Hq, Hkv, d, Lmax, K = 8, 32, 8, 128, 1 << 19, 16
    g = torch.Generator(device=dev)
    g.manual_seed(4321)
    log("[bench] long-context decode: generating 512K-token caches for 8 sequences on device")
    Kc = torch.randn((Bmax, Hkv, Lmax, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    Vc = torch.randn((Bmax, Hkv, Lmax, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    q = torch.randn((Bmax, Hq, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    full = torch.full((Bmax,), Lmax, dtype=torch.int32, device=dev)
    kbar = sas.sas_pool_keys(Kc, full)
    C = Lmax // 64
    s = torch.empty((Bmax, Hkv, C), dtype=torch.float32, device=dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    scale = 1.0 / math.sqrt(d)
    out = []
    for B in (1, 8):
        ws = sas.decode_workspace(B, Hq, Hkv, d, K, dev)
        o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
        for L in (1 << 15, 1 << 17, 1 << 19):
            kv_len = torch.full((B,), L, dtype=torch.int32, device=dev)
            sel_t, att_t = [], []
            for r in range(reps + 3):
                flush.sum()
                a, b_, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                a.record(stream)
                _, idx, cnt, _, _ = sas.sas_decode_select(q[:B], kbar[:B], kv_len, scale, K, s_out=s[:B])
                b_.record(stream)
                sas.sas_decode(q[:B], Kc[:B], Vc[:B], kv_len, idx, cnt, scale, ws=ws, out=o)
                c.record(stream)
                if r >= 3:
                    sel_t.append((a, b_))
                    att_t.append((b_, c))
            torch.cuda.synchronize()
            ms_sel = float(np.median([x.elapsed_time(y) for x, y in sel_t]))
            ms_att = float(np.median([x.elapsed_time(y) for x, y in att_t]))
            ms_two = float(np.median([x[0].elapsed_time(y[1]) for x, y in zip(sel_t, att_t)]))
            # the same step in two launches (sas_decode_long: scores with per-chunk
            # candidates, then the decode ranking them); same output
            wl = sas.decode_long_workspace(B, Hq, Hkv, d, C, K, dev)
            ol = torch.empty_like(o)
            sas.sas_decode_long(q[:B], kbar[:B], Kc[:B], Vc[:B], kv_len, K, scale, ws=wl, out=ol)
            torch.cuda.synchronize()
            assert torch.equal(ol, o), "sas_decode_long differs from sas_decode_select + sas_decode"
            lt = []
            for r in range(reps + 3):
                flush.sum()
                a, c = (torch.cuda.Event(enable_timing=True) for _ in range(2))
                a.record(stream)
                sas.sas_decode_long(q[:B], kbar[:B], Kc[:B], Vc[:B], kv_len, K, scale, ws=wl, out=ol)
                c.record(stream)
                if r >= 3:
                    lt.append((a, c))
            torch.cuda.synchronize()
            ms_long = float(np.median([x.elapsed_time(y) for x, y in lt]))
            hist = (L - 1) // 64
            sel_bytes = B * Hkv * hist * (d * 2 + 4)
            out.append({"context": L, "batch": B, "select_us": round(ms_sel * 1e3, 2),
                        "attn_us": round(ms_att * 1e3, 2),
                        "select_share": round(ms_sel / (ms_sel + ms_att), 3),
                        "select_gbs": round(sel_bytes / ms_sel / 1e6, 1),
                        "step_us": round(ms_two * 1e3, 2),
                        "decode_long_us": round(ms_long * 1e3, 2),
                        # the selection's share of the two-launch step: what the step spends
                        # beyond the attention alone (the same decode, event to event)
                        "decode_long_select_share": round(max(ms_long - ms_att, 0.0) / ms_long, 3)})
            log(f"[bench]   B={B} L={L}: select {ms_sel * 1e3:.1f} us, attention {ms_att * 1e3:.1f} us, "
                f"step {ms_two * 1e3:.1f} us; sas_decode_long {ms_long * 1e3:.1f} us")
    del Kc, Vc, kbar
    return out


def run_sweep(torch, steps, kernel_timing=True):
    """The other prefill configurations, each timed over `steps` steps after 2 warmup
    steps: the 128K-token long prefill (selection + forward, planted scores) and the
    Qwen3-14B-shaped sweep over budgets 16 / 32 / 64 blocks (selection + forward +
    backward with dg, Zipf scores). Q/K/V/dO ~ N(0,1) drawn on the device (seeded)."""
    from learned_context_ranking_amd import sas, synth
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    out = []
    for name in ("long_prefill", "qwen3_14b_k16", "qwen3_14b_k32", "qwen3_14b_k64"):
        w = synth.WORKLOADS[name]
        log(f"[bench] sweep: {name} (generating inputs)")
        g = torch.Generator(device=dev)
        g.manual_seed(99)
        mk = lambda shape: torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        Q, K, V = mk((w.B, w.Hq, w.n, w.d)), mk((w.B, w.Hkv, w.n, w.d)), mk((w.B, w.Hkv, w.n, w.d))
        dO = mk((w.B, w.Hq, w.n, w.d)) if w.backward else None
        s = torch.from_numpy(synth.prefill_scores(w)).to(dev)
        scale = 1.0 / math.sqrt(w.d)
        O = torch.empty_like(Q)
        lse = torch.empty((w.B, w.Hq, w.n), dtype=torch.float32, device=dev)
        if w.backward:
            ws = sas.bwd_workspace(w.B, w.Hq, w.Hkv, w.n, w.d, w.topk, dev)
            outs = (torch.empty(Q.shape, dtype=torch.float32, device=dev),
                    torch.empty(K.shape, dtype=torch.float32, device=dev),
                    torch.empty(V.shape, dtype=torch.float32, device=dev),
                    torch.empty((w.B, w.Hkv, w.NB, w.topk), dtype=torch.float32, device=dev))
        def sweep_step():
            idx, cnt, _, logg = sas.sas_topk_select(s, w.topk, kcap=w.topk, cols=w.NB)
            sas.sas_attn_fwd(Q, K, V, idx, cnt, logg, scale, out=O, lse_out=lse)
            if w.backward:
                sas.sas_attn_bwd(Q, K, V, O, dO, lse, idx, cnt, logg, scale, ws=ws, outs=outs)
            return cnt

        # steps timed with an event pair each and no per-kernel events; the per-kernel
        # breakdown from the same steps run again with every kernel bracketed
        marks = []
        for r in range(steps + 2):
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            cnt = sweep_step()
            b_.record(stream)
            if r >= 2:
                marks.append((a, b_))
        torch.cuda.synchronize()
        prof = {}
        if kernel_timing:
            sas.profile_collect()
            sas.profile_enable(True)
            for _ in range(steps):
                sweep_step()
            torch.cuda.synchronize()
            sas.profile_enable(False)
            prof = sas.profile_collect()
        samples = [x.elapsed_time(y) for x, y in marks]
        ms = float(np.mean(samples))
        pairs = pair_count(cnt.cpu().numpy(), w.G)
        sel_b = select_bytes(w.NB, w.NB, w.B * w.Hkv, w.topk)
        sel_ms = prof["select"][1] / prof["select"][0] if "select" in prof else None
        flop = (12.0 if w.backward else 4.0) * w.d * pairs
        tf = flop / (ms * 1e-3) / 1e12
        out.append({"workload": f"{name}: B={w.B}, Hq={w.Hq}, Hkv={w.Hkv}, d={w.d}, n={w.n}, Top-K={w.topk}, "
                                f"{w.scores} scores, " + ("select+fwd+bwd with dg" if w.backward else "select+fwd"),
                    "ms": round(ms, 4), "tflops": round(tf, 1), "attended_pairs": pairs,
                    "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                    "ms_stats": stats(samples),
                    "select": {"bytes": sel_b, "ms": round(sel_ms, 5) if sel_ms else None,
                               "gbs": round(sel_b / (sel_ms * 1e-3) / 1e9, 1) if sel_ms else None},
                    "kernels_ms": {f"kernel:{k}": round(tot / n, 4) for k, (n, tot) in prof.items()}})
        log(f"[bench]   {name}: {ms:.3f} ms, {tf:.1f} TFLOP/s")
        del Q, K, V, dO, O, s
    return out


def cpu_baseline(w, host, cnt, budget_s=20.0):
    """The oracle (NumPy, float64) on a sample of query blocks of the same workload; FLOPs
    of the sampled blocks over their wall time. Threads = the BLAS pool's size."""
    import oracle
    from learned_context_ranking_amd import synth
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"] or threadpool_info()
        cores = max([p.get("num_threads", 1) for p in info] or [1])
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:   # threadpoolctl missing: report the affinity mask
        cores = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    f = synth.bf16_bits_to_f32
    Q, K, V, dO = f(host["q"]), f(host["k"]), f(host["v"]), f(host["do"])
    idx_r, cnt_r, _, logg_r = oracle.select_prefill(host["s"], w.topk)
    scale = 1.0 / math.sqrt(w.d)
    rng = np.random.default_rng(7)
    t0 = time.perf_counter()
    flops = 0.0
    nblk = 0
    while time.perf_counter() - t0 < budget_s:
        h = int(rng.integers(0, w.Hkv))
        j = int(rng.integers(0, w.NB))
        c = int(cnt_r[0, h, j])
        oracle.fwd_query_block(Q, K, V, 0, h, j, idx_r[0, h, j], c, logg_r[0, h, j], scale)
        oracle.bwd_query_block(Q, K, V, dO, 0, h, j, idx_r[0, h, j], c, logg_r[0, h, j], scale)
        pairs = (64 * 65 // 2 + c * 64 * 64) * w.G
        flops += 12.0 * w.d * pairs
        nblk += 1
    dt = time.perf_counter() - t0
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"{nblk} random (KV head, query block) tiles of the training workload, fwd+bwd "
                       f"with dg, float64 NumPy, {dt:.1f} s wall",
                cpu_model=cpu_model, blas=blas, dtype="f64",
                dtype_reason="the oracle is timed as it stands: it computes in float64 by design (it is "
                             "the parity reference; a float32 run would be a different program)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-decode", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the long-prefill and 14B-sweep configurations")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--decode-reps", type=int, default=200,
                    help="timed decode launches (each after a 1 GiB cache-evicting read)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured MFMA / read peaks")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="time the step without the per-kernel events (no roofline figures)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 256 MiB copy (calibrates the HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the SAS hot path here is a single-GPU library "
              "(heads and batch shard with no communication); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from learned_context_ranking_amd import sas, synth
    from learned_context_ranking_amd.profile_counters import profiled_mfma, profiled_traffic
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    sas.lib()
    if args.calib_copy:
        calibration_copy(torch)
    peaks = None if args.no_peaks else measure_peaks(torch)
    if peaks:
        log(f"[bench] measured peaks: {peaks}")
    w = synth.WORKLOADS["qwen3_4b_train"]
    tr = run_train(w, args.steps, args.warmup, torch, kernel_timing=not args.no_kernel_timing)
    flop_step = tr["flop_fwd"] + tr["flop_bwd"]
    value = flop_step / (tr["ms_step"] * 1e-3) / 1e12
    ms = tr["ms"]
    kern = {"select": ms["sel"], "fwd": ms["fwd"], "bwd": ms["bwd"], "gates_bwd": ms["gates_bwd"],
            "fwd_bwd_gate_outside": ms["fwd_bwd_gate_outside"]}
    kern.update({"kernel:" + k: v for k, v in tr["kern_ms"].items()})
    fwd_tf = tr["flop_fwd"] / (ms["fwd"] * 1e-3) / 1e12
    bwd_tf = tr["flop_bwd"] / (ms["bwd"] * 1e-3) / 1e12
    # Roofline of the dominant kernel (longest average launch), from the library's event
    # timing over the timed region. Algorithmic FLOPs per launch per kernel (pairs = attended
    # (query, key) pairs): fwd 4d (q.k, p.v); dq 4d (dO.v, dS.k); dkv 4d (p^T dO, dS^T q).
    kms = tr["kern_ms"] or {"sas_attn_bwd": ms["bwd"]}
    dom = max(kms, key=kms.get)
    flop_of = {"fwd": 4.0, "dq": 4.0, "dkv": 4.0}
    roof = {"kernel": dom, "bound": "mfma", "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS}
    if dom in flop_of:
        fl = flop_of[dom] * w.d * tr["pairs"]
        roof["flop_per_launch"] = fl
        roof["achieved"] = fl / (kms[dom] * 1e-3) / 1e12
        roof["frac"] = roof["achieved"] / PEAK_BF16_TFLOPS
        if peaks:
            roof["measured_peak"] = peaks["mfma_bf16_tflops"]
            roof["frac_of_measured_peak"] = roof["achieved"] / peaks["mfma_bf16_tflops"]
        if dom in tr["kern_stats"]:
            roof["launch_ms_stats"] = tr["kern_stats"][dom]
    roof["traffic"] = profiled_traffic(dom)
    # matrix-core counters of the same kernel (rocprofv3 MfmaFlopsBF16 / MfmaUtil): the FLOPs
    # it executes (its design recomputes q.k and dO.v) over this run's launch time
    mc = profiled_mfma(dom)
    if mc is not None and dom in kms:
        mc["executed_tflops"] = mc["executed_flop_per_launch"] / (kms[dom] * 1e-3) / 1e12
        mc = {k: round(v, 3) if k != "executed_flop_per_launch" else v for k, v in mc.items()}
    roof["mfma_counters"] = mc
    out = {
        "metric": "gated block-sparse attn TFLOP/s fwd+bwd @n=32K,K=32; decode KV GB/s",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(tr["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "qwen3_4b_train: B=1, Hq=32, Hkv=8, d=128, n=32768, block=64, Top-K=32, "
                        "sparse scope, select+fwd+bwd with dg + score gradient through the gate softmax",
            "global_batch": w.B, "seq_len": w.n, "parallelism": "single GPU",
            "attended_pairs": tr["pairs"], "flop_per_step": flop_step,
        },
        "kernels_ms": {k: round(v, 4) for k, v in kern.items()},
        "step_ms_stats": tr["ev_stats"]["step"],
        "call_ms_stats": {k: v for k, v in tr["ev_stats"].items() if k != "step"},
        "kernel_ms_stats": tr["kern_stats"],
        "select": {"bytes": select_bytes(w.NB, w.NB, w.B * w.Hkv, w.topk),
                   "ms": round(ms["sel"], 5),
                   "gbs": round(select_bytes(w.NB, w.NB, w.B * w.Hkv, w.topk) / (ms["sel"] * 1e-3) / 1e9, 1),
                   "counts": "valid scores read (row j: j of them) + idx/logg (kcap each), cnt, lse written"},
        "measured_peaks": peaks,
        "score_grad_norm": {**{k: round(v, 4) for k, v in tr["gate_grad_norm"].items()},
                            "what": "|ds| over the whole score tensor after select -> fwd -> bwd -> gates_bwd "
                                    "with the history softmax gate vs the kept-set softmax (binary Top-K "
                                    "mask normalisation), same N(0,1) inputs"},
        "fwd_bwd_frac_of_measured_mfma": (round(value / peaks["mfma_bf16_tflops"], 4) if peaks else None),
        "fwd_tflops": round(fwd_tf, 2),
        "bwd_tflops": round(bwd_tf, 2),
        "roofline": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in roof.items()},
    }
    if not args.no_decode:
        dec = run_decode(max(args.steps, args.decode_reps), torch)
        out["decode"] = {"value": round(dec["gbs"], 1), "unit": "GB/s", "ms": round(dec["ms"], 5),
                         "ms_stats": dec["stats"], "bytes": dec["bytes"],
                         "select_ms": round(dec["ms_select"], 5), "select_ms_stats": dec["sel_stats"],
                         "select_bytes": dec["sel_bytes"], "select_gbs": round(dec["sel_gbs"], 1),
                         "end_to_end": {"ms": round(dec["ms_e2e"], 5), "ms_stats": dec["e2e_stats"],
                                        "value": round(dec["e2e_gbs"], 1), "unit": "GB/s",
                                        "counts": "decode bytes + the scores read and idx/cnt/lse written by the "
                                                  "selection, over select + decode time (one step, L2/MALL evicted)"},
                         "steady_state": {"value": round(dec["ss_gbs"], 1), "unit": "GB/s",
                                          "ms_stats": dec["ss_stats"], "bytes": round(dec["ss_bytes"]),
                                          "frac_of_hbm_peak": round(dec["ss_gbs"] / PEAK_HBM_GBS, 4),
                                          "how": "decode steps back to back on the stream (no flush, no host "
                                                 "sync), the selection of 4 score draws in turn so each step's "
                                                 "gather misses the Infinity Cache; per-step event pairs"},
                         "graph_replay": {"value": round(dec["graph_gbs"], 1), "unit": "GB/s",
                                          "ms_stats": dec["graph_stats"], "bytes": round(dec["ss_bytes"]),
                                          "frac_of_hbm_peak": round(dec["graph_gbs"] / PEAK_HBM_GBS, 4),
                                          "how": f"the steady state above captured as {dec['graph_steps']} decode "
                                                 "steps in one HIP graph and replayed (events around each replay, "
                                                 "time / steps); the last step's output checked bit for bit "
                                                 "against an eager launch"},
                         "isolated_launch_note": "value / ms: one launch after a 1 GiB cache-evicting read, "
                                                 "event to event; includes the dispatch latency that a trivial "
                                                 "kernel also shows between two events on this stream",
                         "trivial_kernel_event_ms": round(dec["dispatch_ms"], 5),
                         "fused_select": {
                             "ms": round(dec["ms_fused"], 5), "ms_stats": dec["fused_stats"],
                             "bytes": dec["fused_bytes"],
                             "value": round(dec["fused_bytes"] / dec["ms_fused"] / 1e6, 1),
                             "unit": "GB/s",
                             "steady_state_ms_stats": dec["fss_stats"],
                             "steady_state_value": round((dec["ss_bytes"] + dec["fused_bytes"] - dec["bytes"])
                                                         / dec["fss_ms"] / 1e6, 1),
                             "how": "sas_decode_topk: the Top-K selection inside the decode launch; one launch "
                                    "after the cache-evicting read (compare end_to_end), and steps back to back "
                                    "over 4 score draws (compare steady_state); bytes: the decode's plus the scores read"},
                         "paged": {"ms": round(dec["ms_paged"], 5), "ms_stats": dec["paged_stats"],
                                   "value": round(dec["gbs_paged"], 1),
                                   "unit": "GB/s", "layout": "pool of 64-token pages in random order + page table",
                                   "fused_select": {"ms": round(dec["ms_paged_fused"], 5),
                                                    "ms_stats": dec["paged_fused_stats"],
                                                    "value": round(dec["fused_bytes"] / dec["ms_paged_fused"] / 1e6, 1),
                                                    "unit": "GB/s", "how": "sas_decode_paged_topk, one launch after "
                                                    "the cache-evicting read; bytes as decode.fused_select"}},
                         "early_stop": {f"tau={t}": {"ms": round(v[0], 5), "history_blocks_used": round(v[1], 2)}
                                        for t, v in dec["early"].items()},
                         "workload": dec["workload"],
                         "roofline": {"kernel": "decode", "bound": "hbm", "achieved": round(dec["gbs"], 1),
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": round(dec["gbs"] / PEAK_HBM_GBS, 4),
                                      "frac_of_measured_read": (round(dec["gbs"] / peaks["stream_read_gbs"], 4)
                                                                if peaks else None),
                                      "traffic": profiled_traffic("decode")}}
    if not args.no_long_decode:
        out["long_decode"] = {
            "workload": "one decode step: block scores over pooled keys + Top-K (sas_decode_select), then "
                        "sparse attention (sas_decode); Hq=32, Hkv=8, d=128, K=16 blocks + current block; "
                        "select GB/s counts pooled keys read and scores written; step_us: both, event to "
                        "event; decode_long_us: the same step as sas_decode_long (two launches, same output)",
            "points": run_long_decode(torch)}
    if not args.no_sweep:
        out["sweep"] = run_sweep(torch, args.steps, kernel_timing=not args.no_kernel_timing)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(w, tr["host"], tr["cnt"], args.cpu_seconds)
    props = torch.cuda.get_device_properties(0)
    out["versions"] = {"library": sas.version(), "torch": torch.__version__, "hip": torch.version.hip,
                       "device": props.name, "arch": getattr(props, "gcnArchName", None),
                       "compute_units": props.multi_processor_count}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

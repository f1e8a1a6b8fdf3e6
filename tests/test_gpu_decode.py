"""GPU parity of sas_decode (inference form, Algorithm 2) against the oracle, including
partial current blocks, a sequence with a single token, rows whose budget exceeds their
history, GQA groups of 1, 4, 5 and 8, d = 64 and 128, the gated check variant, and the
full decode workload (64 sequences x 32,768 cached tokens) on sampled sequences, and caches
whose rows past kv_len hold NaN."""
import math

import numpy as np
import pytest
import torch

import oracle
from learned_context_ranking_amd import sas, synth
from gpu_util import assert_close, dev, dev_bf16, host, log

pytestmark = pytest.mark.gpu


def _decode_case(B, Hq, Hkv, d, Lmax, kv_len, topk, seed=0, gated=False, check=None):
    log(f"decode B={B} Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} K={topk} gated={gated}")
    q_bits = synth.normal_bf16((B, Hq, 1, d), seed, synth.TID_QDEC)[:, :, 0]
    k_bits = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_K)
    v_bits = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_V)
    C = (Lmax + 63) // 64
    s = synth.scores_normal((B, Hkv, 1, C), seed)
    kv_len = np.asarray(kv_len, np.int32)
    row_valid = ((kv_len - 1) // 64).astype(np.int32)
    kcap = min(topk, C)
    idx, cnt, _, logg = sas.sas_topk_select(dev(s), topk, mode="decode", row_valid=dev(row_valid), kcap=kcap)
    scale = 1.0 / math.sqrt(d)
    o = sas.sas_decode(dev_bf16(q_bits), dev_bf16(k_bits), dev_bf16(v_bits), dev(kv_len), idx, cnt, scale,
                       logg=logg if gated else None)
    torch.cuda.synchronize()
    idx_r, cnt_r, _, logg_r = oracle.select(s.reshape(B * Hkv, C), np.repeat(row_valid, Hkv), topk, kcap=kcap)
    idx_r = idx_r.reshape(B, Hkv, kcap); cnt_r = cnt_r.reshape(B, Hkv); logg_r = logg_r.reshape(B, Hkv, kcap)
    assert np.array_equal(host(idx)[:, :, 0], idx_r) and np.array_equal(host(cnt)[:, :, 0], cnt_r)
    bs = range(B) if check is None else check
    q = synth.bf16_bits_to_f32(q_bits)
    ref = oracle.decode(q[list(bs)], synth.bf16_bits_to_f32(k_bits[list(bs)]), synth.bf16_bits_to_f32(v_bits[list(bs)]),
                        kv_len[list(bs)], idx_r[list(bs)], cnt_r[list(bs)], scale, logg=logg_r[list(bs)] if gated else None)
    assert_close("o", host(o)[list(bs)], ref)


def test_decode_mixed_lengths():
    _decode_case(4, 8, 2, 128, 4096, [4096, 1000, 65, 1], 8)


def test_decode_gated_variant():
    _decode_case(3, 8, 2, 128, 2048, [2048, 777, 130], 6, gated=True)


@pytest.mark.parametrize("Hq,Hkv,d", [(5, 1, 64), (8, 8, 64), (16, 2, 128), (10, 2, 128), (32, 1, 128),
                                      (64, 2, 64)])
def test_decode_groups(Hq, Hkv, d):
    _decode_case(3, Hq, Hkv, d, 1536, [1536, 900, 64], 5, seed=Hq)


def test_decode_budget_exceeds_history():
    _decode_case(2, 4, 1, 128, 512, [200, 512], 16)


def test_decode_long_list_one_chunk():
    """Lists of 80 blocks + the current one at 512 (sequence, KV head) pairs: the launch
    gives every pair one chunk, so a wave walks 81 list entries and reloads its lane-held
    window of the list after the first 64."""
    B, Hkv = 128, 4
    Lmax = 82 * 64
    kv_len = [Lmax - (b % 7) * 13 for b in range(B)]
    _decode_case(B, 8, Hkv, 64, Lmax, kv_len, 80, seed=3, check=[0, 1, 63, 127])


def test_decode_long_list_small_batch():
    """The same budget at 4 pairs: the lists are split over many chunks and merged."""
    _decode_case(2, 8, 2, 128, 8192, [8192, 5000], 100, seed=4)


def test_decode_full_size():
    """64 sequences, 32 query / 8 KV heads, 32,768 cached tokens, 16 blocks + the current
    one; the oracle checks 4 sampled sequences, the selection is checked on all."""
    _decode_case(64, 32, 8, 128, 32768, [32768] * 64, 16, check=[0, 17, 40, 63])


def _paged_case(B, Hq, Hkv, d, kv_len, topk, seed, npages_extra=37, gated=False):
    """Scatter seeded contiguous caches to random pages of a pool whose other pages (and
    the unused rows of every partial page) hold NaN, then compare with the oracle's paged
    decode and with sas_decode on the contiguous cache."""
    kv_len = np.asarray(kv_len, np.int32)
    maxp = int(-(-kv_len.max() // 64))
    Lmax = maxp * 64
    log(f"paged decode B={B} Hq={Hq} Hkv={Hkv} d={d} kv_len={list(kv_len)} K={topk}")
    q_bits = synth.normal_bf16((B, Hq, 1, d), seed, synth.TID_QDEC)[:, :, 0]
    k_bits = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_K)
    v_bits = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_V)
    g = np.random.default_rng(seed)
    need = [int(-(-L // 64)) for L in kv_len]
    npages = sum(need) + npages_extra
    perm = g.permutation(npages)
    nan = synth.f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    Kp = np.full((npages, Hkv, 64, d), nan, np.uint16)
    Vp = np.full((npages, Hkv, 64, d), nan, np.uint16)
    pt = np.full((B, maxp), -7, np.int32)        # entries past a sequence's blocks are junk
    used = 0
    for b in range(B):
        for m in range(need[b]):
            p = perm[used]; used += 1
            pt[b, m] = p
            rows = min(64, int(kv_len[b]) - 64 * m)
            Kp[p, :, :rows] = k_bits[b, :, 64 * m:64 * m + rows]
            Vp[p, :, :rows] = v_bits[b, :, 64 * m:64 * m + rows]
    C = maxp
    s = synth.scores_normal((B, Hkv, 1, C), seed)
    row_valid = ((kv_len - 1) // 64).astype(np.int32)
    kcap = min(topk, C)
    idx, cnt, _, logg = sas.sas_topk_select(dev(s), topk, mode="decode", row_valid=dev(row_valid), kcap=kcap)
    scale = 1.0 / math.sqrt(d)
    o = sas.sas_decode_paged(dev_bf16(q_bits), dev_bf16(Kp), dev_bf16(Vp), dev(pt), dev(kv_len), idx, cnt, scale,
                             logg=logg if gated else None)
    o_c = sas.sas_decode(dev_bf16(q_bits), dev_bf16(k_bits), dev_bf16(v_bits), dev(kv_len), idx, cnt, scale,
                         logg=logg if gated else None)
    torch.cuda.synchronize()
    idx_r, cnt_r, _, logg_r = oracle.select(s.reshape(B * Hkv, C), np.repeat(row_valid, Hkv), topk, kcap=kcap)
    idx_r = idx_r.reshape(B, Hkv, kcap); cnt_r = cnt_r.reshape(B, Hkv); logg_r = logg_r.reshape(B, Hkv, kcap)
    assert np.array_equal(host(idx)[:, :, 0], idx_r)
    Kf = synth.bf16_bits_to_f32(Kp); Vf = synth.bf16_bits_to_f32(Vp)
    Kf[np.isnan(Kf)] = 0.0; Vf[np.isnan(Vf)] = 0.0      # never read by a correct kernel
    ref = oracle.decode_paged(synth.bf16_bits_to_f32(q_bits), Kf, Vf, pt, kv_len, idx_r, cnt_r, scale,
                              logg=logg_r if gated else None)
    assert_close("o paged", host(o), ref)
    # same arithmetic as the contiguous kernel, block for block
    assert torch.equal(o, o_c)


def test_decode_paged_mixed_lengths():
    _paged_case(5, 8, 2, 128, [4096, 1000, 65, 1, 64 * 20], 8, seed=1)


def test_decode_paged_groups_and_gated():
    _paged_case(3, 10, 2, 128, [1536, 900, 64], 5, seed=2, gated=True)
    _paged_case(2, 5, 1, 64, [777, 130], 4, seed=3)


def test_decode_paged_large_batch():
    """64 sequences (one chunk per (sequence, KV head), the direct-output path)."""
    _paged_case(64, 32, 8, 128, [4096 - 13 * b for b in range(64)], 16, seed=4, npages_extra=5)


def _early_case(B, Hq, Hkv, d, Lmax, kv_len, topk, taus, seed):
    """Early-stopped decode against the oracle: the order key is the selection score
    itself (exact on both sides); for each tau, heads whose every stop comparison is far
    from the threshold (the oracle reports the margin) must use the same number of
    blocks and give the same output."""
    log(f"early-stop decode B={B} Hq={Hq} Hkv={Hkv} d={d} K={topk} taus={taus}")
    q_bits = synth.normal_bf16((B, Hq, 1, d), seed, synth.TID_QDEC)[:, :, 0]
    k_bits = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_K)
    v_bits = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_V)
    C = (Lmax + 63) // 64
    s = synth.scores_normal((B, Hkv, 1, C), seed)
    kv_len = np.asarray(kv_len, np.int32)
    row_valid = ((kv_len - 1) // 64).astype(np.int32)
    kcap = min(topk, C)
    idx_r, cnt_r, _, _ = oracle.select(s.reshape(B * Hkv, C), np.repeat(row_valid, Hkv), topk, kcap=kcap)
    idx_r = idx_r.reshape(B, Hkv, kcap); cnt_r = cnt_r.reshape(B, Hkv)
    order = np.zeros((B, Hkv, kcap), np.float32)
    for b in range(B):
        for h in range(Hkv):
            c = cnt_r[b, h]
            order[b, h, :c] = s[b, h, 0, idx_r[b, h, :c]]
    Q, K, V = dev_bf16(q_bits), dev_bf16(k_bits), dev_bf16(v_bits)
    idx, cnt = dev(idx_r), dev(cnt_r)
    scale = 1.0 / math.sqrt(d)
    qf, Kf, Vf = (synth.bf16_bits_to_f32(x) for x in (q_bits, k_bits, v_bits))
    for tau in taus:
        o, used = sas.sas_decode_early_stop(Q, K, V, dev(kv_len), idx, cnt, dev(order), scale, tau)
        torch.cuda.synchronize()
        o_r, used_r, _ = oracle.decode_early_stop(qf, Kf, Vf, kv_len, idx_r, cnt_r, order, scale, tau)
        ug, og = host(used), host(o)
        # per-head margins: recompute each head alone to know whether its decisions are safe
        safe = np.zeros((B, Hq), bool)
        G = Hq // Hkv
        for b in range(B):
            for hq in range(Hq):
                h = hq // G
                _, _, mg = oracle.decode_early_stop(qf[b:b + 1, hq:hq + 1], Kf[b:b + 1, h:h + 1], Vf[b:b + 1, h:h + 1],
                                                    kv_len[b:b + 1], idx_r[b:b + 1, h:h + 1], cnt_r[b:b + 1, h:h + 1],
                                                    order[b:b + 1, h:h + 1], scale, tau)
                safe[b, hq] = mg > 1e-3
        cnt_q = np.repeat(cnt_r, G, axis=1)
        assert np.all((ug >= np.minimum(cnt_q, 1)) & (ug <= cnt_q))
        assert np.array_equal(ug[safe], used_r[safe]), tau
        log(f"  tau={tau}: blocks used mean {ug.mean():.2f} of {cnt_q.mean():.2f}; {safe.mean():.0%} heads compared")
        if safe.any():
            assert_close(f"o early stop tau={tau}", og[safe], o_r[safe])
        if tau == 0.0:
            assert np.array_equal(ug, cnt_q)
            assert_close("o tau=0 vs oracle decode", og, oracle.decode(qf, Kf, Vf, kv_len, idx_r, cnt_r, scale))


def test_decode_early_stop_thresholds():
    _early_case(4, 8, 2, 128, 4096, [4096, 1000, 65, 64 * 40 + 7], 16, [0.0, 1e-3, 0.01, 0.05, 0.5], seed=7)


def test_decode_early_stop_groups_small_d():
    _early_case(3, 5, 1, 64, 2048, [2048, 777, 130], 12, [0.0, 0.02], seed=8)
    _early_case(2, 32, 8, 128, 64 * 100, [6400, 3000], 63, [0.005, 0.1], seed=9)


def test_decode_permuted_workgroup_order():
    """Decode output is bit-identical when the workgroups take their chunks in a permuted
    order (split lists are merged in chunk order)."""
    B, Hq, Hkv, d, Lmax, topk = 3, 8, 2, 128, 4096, 24
    q_bits = synth.normal_bf16((B, Hq, 1, d), 5, synth.TID_QDEC)[:, :, 0]
    k_bits = synth.normal_bf16((B, Hkv, Lmax, d), 5, synth.TID_K)
    v_bits = synth.normal_bf16((B, Hkv, Lmax, d), 5, synth.TID_V)
    s = synth.scores_normal((B, Hkv, 1, Lmax // 64), 5)
    kv_len = np.array([4096, 2500, 700], np.int32)
    rv = ((kv_len - 1) // 64).astype(np.int32)
    idx, cnt, _, _ = sas.sas_topk_select(dev(s), topk, mode="decode", row_valid=dev(rv), kcap=topk)
    q, K, V, L = dev_bf16(q_bits), dev_bf16(k_bits), dev_bf16(v_bits), dev(kv_len)
    o0 = sas.sas_decode(q, K, V, L, idx, cnt, 1.0 / math.sqrt(d))
    try:
        sas.debug_workgroup_order(99)
        o1 = sas.sas_decode(q, K, V, L, idx, cnt, 1.0 / math.sqrt(d))
    finally:
        sas.debug_workgroup_order(0)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)


def test_decode_ignores_rows_past_kv_len():
    """Cache rows at or past kv_len (the rest of the current block and beyond) hold NaN:
    they are never used, so decode, early-stopped decode (tau = 0: every kept block) and
    the decode with its selection all match the oracle, which reads only the valid rows."""
    B, Hq, Hkv, d, Lmax, topk = 4, 8, 2, 128, 2048, 8
    kv_len = np.array([2048, 1000, 65, 1], np.int32)
    log(f"decode with NaN past kv_len B={B} Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} K={topk}")
    q_bits = synth.normal_bf16((B, Hq, 1, d), 7, synth.TID_QDEC)[:, :, 0]
    k_bits = synth.normal_bf16((B, Hkv, Lmax, d), 7, synth.TID_K)
    v_bits = synth.normal_bf16((B, Hkv, Lmax, d), 7, synth.TID_V)
    for b in range(B):
        k_bits[b, :, kv_len[b]:] = 0x7FC0   # bf16 quiet NaN
        v_bits[b, :, kv_len[b]:] = 0x7FC0
    C = Lmax // 64
    s = synth.scores_normal((B, Hkv, 1, C), 7)
    row_valid = ((kv_len - 1) // 64).astype(np.int32)
    scale = 1.0 / math.sqrt(d)
    q, Kc, Vc, kvl, sd = dev_bf16(q_bits), dev_bf16(k_bits), dev_bf16(v_bits), dev(kv_len), dev(s)
    idx, cnt, _, _ = sas.sas_topk_select(sd, topk, mode="decode", row_valid=dev(row_valid), kcap=topk)
    idx3, cnt3 = idx.reshape(B, Hkv, topk), cnt.reshape(B, Hkv)
    o = sas.sas_decode(q, Kc, Vc, kvl, idx, cnt, scale)
    of = sas.sas_decode_topk(q, Kc, Vc, kvl, sd, topk, scale)
    order = torch.gather(sd[:, :, 0, :], -1, idx3.clamp(min=0).long()).contiguous()
    oe, _ = sas.sas_decode_early_stop(q, Kc, Vc, kvl, idx3.contiguous(), cnt3.contiguous(), order, scale, 0.0)
    torch.cuda.synchronize()
    idx_r, cnt_r, _, _ = oracle.select(s.reshape(B * Hkv, C), np.repeat(row_valid, Hkv), topk, kcap=topk)
    ref = oracle.decode(synth.bf16_bits_to_f32(q_bits), synth.bf16_bits_to_f32(k_bits),
                        synth.bf16_bits_to_f32(v_bits), kv_len, idx_r.reshape(B, Hkv, topk),
                        cnt_r.reshape(B, Hkv), scale)
    assert_close("o (decode)", host(o), ref)
    assert_close("o (decode_topk)", host(of), ref)
    assert_close("o (early stop, tau 0)", host(oe), ref)

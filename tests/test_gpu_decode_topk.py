"""GPU parity of sas_decode_topk: one decode step with its block selection in the same launch
([SAS-ja] "仕組み", Algorithm 2). The kept blocks must equal sas_topk_select's in decode mode
and the oracle's selection exactly. The output must equal sas_topk_select followed by
sas_decode bit for bit, and the oracle's decode within the decode tolerance. Cases: the full
decode workload, mixed and very short sequences (no history, budget above history), d = 64,
GQA groups of 4 and 5, a small batch whose lists are split over several workgroups, and
scores with ties, NaN, -inf and -0. sas_decode_paged_topk (the same over a paged cache) must
equal sas_topk_select + sas_decode_paged and the contiguous form bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle
from learned_context_ranking_amd import sas, synth
from gpu_util import assert_close, dev, dev_bf16, host, log

pytestmark = pytest.mark.gpu


def _scores(B, Hkv, C, seed, kind):
    s = synth.scores_normal((B, Hkv, 1, C), seed)
    if kind == "const":
        s = np.full_like(s, 0.25)                      # every key equal: the K lowest indices
    if kind == "ties":
        s = np.round(s * 2.0) / 2.0                    # few distinct values: many ties at the cut
        s[..., 3::7] = np.nan
        s[..., 5::11] = -np.inf
        s[..., 1::13] = -0.0
        s[..., 2::17] = 0.0
    return np.ascontiguousarray(s.astype(np.float32))


def _case(B, Hq, Hkv, d, Lmax, kv_len, topk, seed=0, kind="normal", check=None):
    log(f"decode_topk B={B} Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} K={topk} scores={kind}")
    q_bits = synth.normal_bf16((B, Hq, 1, d), seed, synth.TID_QDEC)[:, :, 0]
    k_bits = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_K)
    v_bits = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_V)
    C = (Lmax + 63) // 64
    s = _scores(B, Hkv, C, seed, kind)
    kv_len = np.asarray(kv_len, np.int32)
    row_valid = ((kv_len - 1) // 64).astype(np.int32)
    scale = 1.0 / math.sqrt(d)
    q, Kc, Vc, kvl, sd = dev_bf16(q_bits), dev_bf16(k_bits), dev_bf16(v_bits), dev(kv_len), dev(s)

    o, idx, cnt = sas.sas_decode_topk(q, Kc, Vc, kvl, sd, topk, scale, want_idx=True)
    idx2, cnt2, _, _ = sas.sas_topk_select(sd, topk, mode="decode", row_valid=dev(row_valid), kcap=topk)
    o2 = sas.sas_decode(q, Kc, Vc, kvl, idx2, cnt2, scale)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), host(idx2)[:, :, 0]) and np.array_equal(host(cnt), host(cnt2)[:, :, 0])
    assert torch.equal(o, o2), "fused and two-step decode differ"

    idx_r, cnt_r, _, _ = oracle.select(s.reshape(B * Hkv, C), np.repeat(row_valid, Hkv), topk, kcap=topk)
    idx_r = idx_r.reshape(B, Hkv, topk); cnt_r = cnt_r.reshape(B, Hkv)
    assert np.array_equal(host(idx), idx_r) and np.array_equal(host(cnt), cnt_r)
    bs = list(range(B)) if check is None else check
    ref = oracle.decode(synth.bf16_bits_to_f32(q_bits)[bs], synth.bf16_bits_to_f32(k_bits[bs]),
                        synth.bf16_bits_to_f32(v_bits[bs]), kv_len[bs], idx_r[bs], cnt_r[bs], scale)
    assert_close("o", host(o)[bs], ref)


def test_decode_topk_full_size():
    """64 sequences, 32 query / 8 KV heads, 32,768 cached tokens, K = 16: every pair one
    workgroup; the oracle checks 4 sampled sequences, everything else is checked on all."""
    _case(64, 32, 8, 128, 32768, [32768] * 64, 16, check=[0, 21, 42, 63])


def test_decode_topk_mixed_lengths_d64():
    """No history (1 and 64 tokens), a partial current block, budget above history."""
    _case(6, 8, 2, 64, 4096, [4096, 1000, 65, 1, 64, 129], 8, seed=1)


def test_decode_topk_split_lists():
    """4 (sequence, KV head) pairs with K = 64: each list is split over several workgroups,
    every one of which selects the row again, and the partial states are merged."""
    _case(2, 8, 2, 128, 16384, [16384, 9000], 64, seed=2)


def test_decode_topk_group_of_five():
    _case(3, 10, 2, 128, 2048, [2048, 1500, 700], 12, seed=3)


def test_decode_topk_group_of_32():
    """The largest group: 32 query heads per KV head fill the 32 query columns of the tile."""
    _case(3, 32, 1, 128, 4096, [4096, 2500, 300], 16, seed=7)


def test_decode_topk_ties_nan():
    """Scores on a half-integer grid (ties at the cut broken toward the lower index), NaN and
    -inf ranked lowest, -0 equal to +0."""
    _case(4, 8, 4, 128, 8192, [8192, 8000, 3000, 640], 24, seed=4, kind="ties")


def test_decode_topk_budget_above_history():
    """K = 32 over 16 history blocks at most: every history block is kept, -1 padded."""
    _case(2, 4, 1, 128, 1024, [1024, 300], 32, seed=5)


def test_decode_topk_all_equal():
    """Every score equal: the cut is that key, and the walk keeps its K lowest indices."""
    _case(3, 8, 2, 64, 4096, [4096, 2000, 700], 20, seed=6, kind="const")


def _paged(Kc, Vc, seed):
    """The caches as a pool of 64-token pages in random order plus a page table."""
    B, Hkv, Lmax, d = Kc.shape
    C = Lmax // 64
    perm = torch.randperm(B * C, generator=torch.Generator().manual_seed(seed)).to(Kc.device)
    Kp = Kc.reshape(B, Hkv, C, 64, d).permute(0, 2, 1, 3, 4).reshape(B * C, Hkv, 64, d)[perm].contiguous()
    Vp = Vc.reshape(B, Hkv, C, 64, d).permute(0, 2, 1, 3, 4).reshape(B * C, Hkv, 64, d)[perm].contiguous()
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(B * C, device=perm.device)
    return Kp, Vp, inv.reshape(B, C).to(torch.int32).contiguous()


@pytest.mark.parametrize("B,Hq,Hkv,d,Lmax,kv_len,topk", [
    (4, 8, 2, 128, 4096, [4096, 1000, 65, 1], 8),
    (2, 8, 2, 64, 8192, [8192, 5000], 64),
    (64, 32, 8, 128, 2048, None, 16),
], ids=["mixed", "split-lists-d64", "one-chunk"])
def test_decode_paged_topk(B, Hq, Hkv, d, Lmax, kv_len, topk):
    """Paged caches (pages in random order): kept blocks and output equal to
    sas_topk_select + sas_decode_paged and to the contiguous sas_decode_topk, bit for bit;
    output against the oracle. Rows of the current page past kv_len hold NaN."""
    log(f"decode_paged_topk B={B} Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} K={topk}")
    seed = 8
    kv_len = np.asarray(kv_len if kv_len is not None else [Lmax - 37 * (b % 5) for b in range(B)], np.int32)
    q_bits = synth.normal_bf16((B, Hq, 1, d), seed, synth.TID_QDEC)[:, :, 0]
    k_bits = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_K)
    v_bits = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_V)
    for b in range(B):
        k_bits[b, :, kv_len[b]:] = 0x7FC0
        v_bits[b, :, kv_len[b]:] = 0x7FC0
    C = Lmax // 64
    s = synth.scores_normal((B, Hkv, 1, C), seed)
    row_valid = ((kv_len - 1) // 64).astype(np.int32)
    scale = 1.0 / math.sqrt(d)
    q, Kc, Vc, kvl, sd = dev_bf16(q_bits), dev_bf16(k_bits), dev_bf16(v_bits), dev(kv_len), dev(s)
    Kp, Vp, pt = _paged(Kc, Vc, seed)

    o, idx, cnt = sas.sas_decode_paged_topk(q, Kp, Vp, pt, kvl, sd, topk, scale, want_idx=True)
    idx2, cnt2, _, _ = sas.sas_topk_select(sd, topk, mode="decode", row_valid=dev(row_valid), kcap=topk)
    o2 = sas.sas_decode_paged(q, Kp, Vp, pt, kvl, idx2.reshape(B, Hkv, topk), cnt2.reshape(B, Hkv), scale)
    o3 = sas.sas_decode_topk(q, Kc, Vc, kvl, sd, topk, scale)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), host(idx2)[:, :, 0]) and np.array_equal(host(cnt), host(cnt2)[:, :, 0])
    assert torch.equal(o, o2), "fused and two-step paged decode differ"
    assert torch.equal(o, o3), "paged and contiguous fused decode differ"
    idx_r, cnt_r, _, _ = oracle.select(s.reshape(B * Hkv, C), np.repeat(row_valid, Hkv), topk, kcap=topk)
    bs = list(range(min(B, 6)))
    ref = oracle.decode(synth.bf16_bits_to_f32(q_bits)[bs], synth.bf16_bits_to_f32(k_bits[bs]),
                        synth.bf16_bits_to_f32(v_bits[bs]), kv_len[bs], idx_r.reshape(B, Hkv, topk)[bs],
                        cnt_r.reshape(B, Hkv)[bs], scale)
    assert_close("o", host(o)[bs], ref)


def test_decode_paged_topk_bad_current_page():
    """A current page id outside the pool reads nothing: that block has weight 0, the kept
    history blocks still count, and the result equals the two-step paged decode."""
    B, Hq, Hkv, d, Lmax, topk = 2, 8, 2, 128, 2048, 8
    log(f"decode_paged_topk bad current page B={B} Lmax={Lmax} K={topk}")
    kv_len = np.array([2048, 1500], np.int32)
    q = dev_bf16(synth.normal_bf16((B, Hq, 1, d), 9, synth.TID_QDEC)[:, :, 0])
    Kc = dev_bf16(synth.normal_bf16((B, Hkv, Lmax, d), 9, synth.TID_K))
    Vc = dev_bf16(synth.normal_bf16((B, Hkv, Lmax, d), 9, synth.TID_V))
    s = dev(synth.scores_normal((B, Hkv, 1, Lmax // 64), 9))
    Kp, Vp, pt = _paged(Kc, Vc, 9)
    for b in range(B):
        pt[b, (int(kv_len[b]) - 1) // 64] = -3 if b == 0 else Kp.shape[0]   # negative, and one past the pool
    kvl = dev(kv_len)
    scale = 1.0 / math.sqrt(d)
    o = sas.sas_decode_paged_topk(q, Kp, Vp, pt, kvl, s, topk, scale)
    row_valid = dev(((kv_len - 1) // 64).astype(np.int32))
    idx, cnt, _, _ = sas.sas_topk_select(s, topk, mode="decode", row_valid=row_valid, kcap=topk)
    o2 = sas.sas_decode_paged(q, Kp, Vp, pt, kvl, idx.reshape(B, Hkv, topk), cnt.reshape(B, Hkv), scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    assert torch.equal(o, o2)

"""GPU parity of sas_decode_topk: one decode step with its block selection in the same launch
([SAS-ja] "仕組み", Algorithm 2). The kept blocks must equal sas_topk_select's in decode mode
and the oracle's selection exactly. The output must equal sas_topk_select followed by
sas_decode bit for bit, and the oracle's decode within the decode tolerance. Cases: the full
decode workload, mixed and very short sequences (no history, budget above history), d = 64,
GQA groups of 4 and 5, a small batch whose lists are split over several workgroups, and
scores with ties, NaN, -inf and -0."""
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

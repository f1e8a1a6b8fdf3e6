"""GPU parity of sas_decode (inference form, Algorithm 2) against the oracle, including
partial current blocks, a sequence with a single token, rows whose budget exceeds their
history, GQA groups of 1, 4, 5 and 8, d = 64 and 128, the gated check variant, and the
full decode workload (64 sequences x 32,768 cached tokens) on sampled sequences."""
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


@pytest.mark.parametrize("Hq,Hkv,d", [(5, 1, 64), (8, 8, 64), (16, 2, 128), (10, 2, 128)])
def test_decode_groups(Hq, Hkv, d):
    _decode_case(3, Hq, Hkv, d, 1536, [1536, 900, 64], 5, seed=Hq)


def test_decode_budget_exceeds_history():
    _decode_case(2, 4, 1, 128, 512, [200, 512], 16)


def test_decode_full_size():
    """64 sequences, 32 query / 8 KV heads, 32,768 cached tokens, 16 blocks + the current
    one; the oracle checks 4 sampled sequences, the selection is checked on all."""
    _decode_case(64, 32, 8, 128, 32768, [32768] * 64, 16, check=[0, 17, 40, 63])

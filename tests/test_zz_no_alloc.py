"""sas_decode_noalloc: the decode entry point that allocates nothing (its partial softmax
states go to the library's per-device scratch) against sas_decode with a caller workspace,
on two calls in a row (the second smaller, so it reuses scratch the first one wrote), plus
the oracle on the first. Both cases split every list over several workgroups, so the
scratch carries the partial states."""
import math

import numpy as np
import pytest
import torch

import oracle
from learned_context_ranking_amd import sas, synth
from gpu_util import assert_close, dev, dev_bf16, host, log

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, d, Lmax, kv_len, topk, seed):
    q_bits = synth.normal_bf16((B, Hq, 1, d), seed, synth.TID_QDEC)[:, :, 0]
    k_bits = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_K)
    v_bits = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_V)
    C = Lmax // 64
    s = synth.scores_normal((B, Hkv, 1, C), seed)
    kv_len = np.asarray(kv_len, np.int32)
    rv = ((kv_len - 1) // 64).astype(np.int32)
    kcap = min(topk, C)
    return q_bits, k_bits, v_bits, s, kv_len, rv, kcap


def _split_lists(B, Hkv, kcap):
    # the launch splits each (sequence, KV head) list when fewer than 512 pairs fill the chip
    return B * Hkv < 512 and kcap + 1 >= 3


def test_noalloc_matches_decode_on_two_calls():
    scale128, scale64 = 1.0 / math.sqrt(128), 1.0 / math.sqrt(64)
    cases = [(4, 8, 2, 128, 4096, [4096, 3000, 130, 64], 16, 11, scale128),
             (2, 8, 2, 64, 2048, [2048, 777], 8, 12, scale64)]
    for i, (B, Hq, Hkv, d, Lmax, kvl, topk, seed, scale) in enumerate(cases):
        log(f"noalloc call {i}: B={B} Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} K={topk}")
        qb, kb, vb, s, kv_len, rv, kcap = _inputs(B, Hq, Hkv, d, Lmax, kvl, topk, seed)
        assert _split_lists(B, Hkv, kcap)
        idx, cnt, _, _ = sas.sas_topk_select(dev(s), topk, mode="decode", row_valid=dev(rv), kcap=kcap)
        q, K, V, L = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev(kv_len)
        o_ws = sas.sas_decode(q, K, V, L, idx, cnt, scale)
        o_na = torch.full_like(o_ws, float("nan"))
        sas.sas_decode_noalloc(q, K, V, L, idx, cnt, scale, out=o_na)
        torch.cuda.synchronize()
        # the same kernels and the same chunking: bit-identical to the workspace path
        assert torch.equal(o_na, o_ws), f"call {i}: noalloc output differs from sas_decode"
        if i == 0:
            idx_r, cnt_r, _, _ = oracle.select(s.reshape(B * Hkv, -1), np.repeat(rv, Hkv), topk, kcap=kcap)
            ref = oracle.decode(synth.bf16_bits_to_f32(qb), synth.bf16_bits_to_f32(kb), synth.bf16_bits_to_f32(vb),
                                kv_len, idx_r.reshape(B, Hkv, kcap), cnt_r.reshape(B, Hkv), scale)
            assert_close("o (noalloc)", host(o_na), ref)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    """511 (sequence, KV head) pairs with 32 query heads each and d = 128 would need 2 chunks
    per list and ~17 MB of partial states, beyond the 16 MiB scratch: rejected, nothing
    launched (the output keeps its contents)."""
    B, Hq, Hkv, d, Lmax, kcap = 511, 32, 1, 128, 256, 3
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((B, Hkv, Lmax, d), dtype=torch.bfloat16, device="cuda")
    L = torch.full((B,), Lmax, dtype=torch.int32, device="cuda")
    idx = torch.zeros((B, Hkv, kcap), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    o = torch.full_like(q, 7.0)
    with pytest.raises(sas.SasError) as e:
        sas.sas_decode_noalloc(q, K, K, L, idx, cnt, 0.1, out=o)
    assert e.value.status == sas.SAS_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())

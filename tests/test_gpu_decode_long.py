"""GPU parity of sas_decode_long: one long-context decode step (block scores over the pooled
keys, Top-K, decode; [SAS-ja] "仕組み" Algorithm 2 with the block score of [PBS-ja] sections
3 and 4) in two launches.

* Against the three-launch path, sas_decode_select (kcap = K) then sas_decode, on the same
  device inputs: kept blocks, counts and output bit for bit. Contexts from 8K to 512K
  tokens (C up to 8192 pooled blocks), K = 16 and 64 (so the candidate chunks take 128 to
  512 blocks), d = 64 and 128, GQA groups of 4 and 5, mixed lengths down to no history.
* Exact integer keys and queries repeating with a short period: every score is exact in
  fp32 and in the oracle's float64 and the K-th score of each row is tied, so the kept
  blocks equal the oracle's decode_select bit for bit and the output the oracle's decode.
* Paged caches (sas_pool_keys_paged, sas_decode_long_paged) with pages in random order:
  pooled keys, kept blocks and output equal to the contiguous path bit for bit; an
  out-of-range page id pools to zero.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from learned_context_ranking_amd import sas, synth
from gpu_util import assert_close, dev, dev_bf16, host, log

pytestmark = pytest.mark.gpu


def _compare_paths(q, Kc, Vc, kbar, kv_len, topk, scale):
    B, Hkv = Kc.shape[0], Kc.shape[1]
    o, idx, cnt = sas.sas_decode_long(q, kbar, Kc, Vc, kv_len, topk, scale, want_idx=True)
    s = torch.empty((B, Hkv, kbar.shape[2]), dtype=torch.float32, device=q.device)
    _, idx2, cnt2, _, _ = sas.sas_decode_select(q, kbar, kv_len, scale, topk, kcap=topk, s_out=s)
    o2 = sas.sas_decode(q, Kc, Vc, kv_len, idx2, cnt2, scale)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2.reshape(idx.shape)), "kept blocks differ from sas_decode_select"
    assert torch.equal(cnt, cnt2.reshape(cnt.shape))
    assert torch.equal(o, o2), "output differs from sas_decode_select + sas_decode"
    return o, idx, cnt


@pytest.mark.parametrize("B,Hq,Hkv,d,Lmax,topk", [
    (2, 8, 2, 128, 8192, 16),
    (1, 32, 8, 128, 131072, 16),
    (1, 32, 8, 128, 131072, 64),
    (3, 10, 2, 64, 65536, 32),
    (8, 32, 8, 128, 32768, 16),
    (2, 64, 2, 64, 16384, 16),
], ids=["8K", "128K-K16", "128K-K64", "64K-d64-G5", "32K-B8", "16K-d64-G32"])
def test_decode_long_matches_select_then_decode(B, Hq, Hkv, d, Lmax, topk):
    log(f"decode_long B={B} Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} K={topk}")
    g = torch.Generator(device="cuda")
    g.manual_seed(Lmax + topk + d)
    Kc = torch.randn((B, Hkv, Lmax, d), generator=g, device="cuda").to(torch.bfloat16)
    Vc = torch.randn((B, Hkv, Lmax, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    lens = [Lmax, Lmax - 777, 64 * 40 + 3, 1, 65, Lmax // 3, 129, Lmax - 64]
    kv_len = dev(np.array(lens[:B], np.int32))
    kbar = sas.sas_pool_keys(Kc, kv_len)
    _compare_paths(q, Kc, Vc, kbar, kv_len, topk, 1.0 / math.sqrt(d))


def test_decode_long_512k():
    """The longest context of the pages' decode measurement: 512K tokens, C = 8192 pooled
    blocks (8191 history blocks), K = 16 (candidate chunks of 128 blocks) and K = 64 (512)."""
    B, Hq, Hkv, d, Lmax = 1, 32, 8, 128, 524288
    log(f"decode_long 512K B={B} Hq={Hq} Hkv={Hkv} d={d}")
    g = torch.Generator(device="cuda")
    g.manual_seed(512)
    Kc = torch.randn((B, Hkv, Lmax, d), generator=g, device="cuda").to(torch.bfloat16)
    Vc = torch.randn((B, Hkv, Lmax, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    kv_len = dev(np.array([Lmax], np.int32))
    kbar = sas.sas_pool_keys(Kc, kv_len)
    for topk in (16, 64):
        _compare_paths(q, Kc, Vc, kbar, kv_len, topk, 1.0 / math.sqrt(d))


def _int_bits(shape, seed, lo=-2, hi=2):
    g = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits(g.integers(lo, hi + 1, size=shape).astype(np.float32))


@pytest.mark.parametrize("Hq,Hkv,d,period,topk", [(8, 2, 128, 5, 16), (10, 2, 64, 7, 24)])
def test_decode_long_exact_ties_against_oracle(Hq, Hkv, d, period, topk):
    """Integer keys repeating every `period` blocks (so each row has `period` distinct
    scores and ties at its K-th), integer queries, scale 1/8: exact on both sides."""
    log(f"decode_long exact ties Hq={Hq} Hkv={Hkv} d={d} period={period} K={topk}")
    B, Lmax = 3, 64 * 300
    kb = _int_bits((B, Hkv, 64 * period, d), Hq + d)
    reps = -(-Lmax // (64 * period))
    kb = np.ascontiguousarray(np.tile(kb, (1, 1, reps, 1))[:, :, :Lmax])
    vb = synth.normal_bf16((B, Hkv, Lmax, d), 11, synth.TID_V)
    qb = _int_bits((B, Hq, d), Hq + d + 1)
    kv_len = np.array([Lmax, 64 * 131 + 5, 64 * 9], np.int32)
    scale = 0.125
    q, Kc, Vc, kvl = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev(kv_len)
    kbar = sas.sas_pool_keys(Kc, kvl)
    o, idx, cnt = _compare_paths(q, Kc, Vc, kbar, kvl, topk, scale)
    kf, qf = synth.bf16_bits_to_f32(kb), synth.bf16_bits_to_f32(qb)
    _, idx_r, cnt_r, _, _ = oracle.decode_select(qf, kf, kv_len, scale, topk, kcap=topk)
    assert np.array_equal(host(idx), idx_r) and np.array_equal(host(cnt), cnt_r)
    ref = oracle.decode(qf, kf, synth.bf16_bits_to_f32(vb), kv_len, idx_r, cnt_r, scale)
    assert_close("o", host(o), ref)


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


@pytest.mark.parametrize("B,Hq,Hkv,d,Lmax,topk", [
    (3, 8, 2, 128, 65536, 16),
    (2, 10, 2, 64, 32768, 64),
], ids=["64K-K16", "32K-d64-G5-K64"])
def test_decode_long_paged_matches_contiguous(B, Hq, Hkv, d, Lmax, topk):
    """Pages in random order: pooled keys equal to sas_pool_keys on the contiguous cache, and
    kept blocks and output equal to sas_decode_long on it (so to sas_decode_select +
    sas_decode_paged), bit for bit."""
    log(f"decode_long_paged B={B} Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} K={topk}")
    g = torch.Generator(device="cuda")
    g.manual_seed(Lmax + d)
    Kc = torch.randn((B, Hkv, Lmax, d), generator=g, device="cuda").to(torch.bfloat16)
    Vc = torch.randn((B, Hkv, Lmax, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    kv_len = dev(np.array([Lmax, Lmax // 2 + 7, 200][:B], np.int32))
    Kp, Vp, pt = _paged(Kc, Vc, 21)
    scale = 1.0 / math.sqrt(d)
    kbar = sas.sas_pool_keys(Kc, kv_len)
    kbar_p = sas.sas_pool_keys_paged(Kp, pt, kv_len)
    o, idx, cnt = sas.sas_decode_long(q, kbar, Kc, Vc, kv_len, topk, scale, want_idx=True)
    op, idxp, cntp = sas.sas_decode_long_paged(q, kbar_p, Kp, Vp, pt, kv_len, topk, scale, want_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(kbar_p, kbar), "paged pooled keys differ"
    assert torch.equal(idxp, idx) and torch.equal(cntp, cnt)
    assert torch.equal(op, o), "paged and contiguous long decode differ"


def test_pool_keys_paged_bad_page():
    """A page id outside the pool pools to zero; the other blocks are unchanged."""
    B, Hkv, d, Lmax = 2, 2, 128, 4096
    log(f"pool_keys_paged bad page B={B} Hkv={Hkv} d={d} Lmax={Lmax}")
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    Kc = torch.randn((B, Hkv, Lmax, d), generator=g, device="cuda").to(torch.bfloat16)
    Kp, _, pt = _paged(Kc, Kc, 6)
    kv_len = dev(np.array([Lmax, Lmax], np.int32))
    pt[0, 3] = -1
    pt[1, 10] = Kp.shape[0]
    kbar = sas.sas_pool_keys(Kc, kv_len)
    kbar_p = sas.sas_pool_keys_paged(Kp, pt, kv_len)
    torch.cuda.synchronize()
    assert torch.all(kbar_p[0, :, 3] == 0) and torch.all(kbar_p[1, :, 10] == 0)
    kbar[0, :, 3] = 0
    kbar[1, :, 10] = 0
    assert torch.equal(kbar_p, kbar)


def test_decode_long_kv_len_past_cache_is_clamped():
    """kv_len above Lmax reads as Lmax (the documented clamp) in both launches: kept blocks,
    counts and output equal those of kv_len = Lmax, and no kept block is the current one."""
    B, Hq, Hkv, d, Lmax, topk = 2, 8, 2, 128, 4096, 16
    log(f"decode_long kv_len past the cache B={B} Lmax={Lmax} K={topk}")
    g = torch.Generator(device="cuda")
    g.manual_seed(33)
    Kc = torch.randn((B, Hkv, Lmax, d), generator=g, device="cuda").to(torch.bfloat16)
    Vc = torch.randn((B, Hkv, Lmax, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    full = dev(np.array([Lmax, Lmax], np.int32))
    kbar = sas.sas_pool_keys(Kc, full)              # every block pooled, the last one too
    scale = 1.0 / math.sqrt(d)
    o, idx, cnt = sas.sas_decode_long(q, kbar, Kc, Vc, full, topk, scale, want_idx=True)
    o2, idx2, cnt2 = sas.sas_decode_long(q, kbar, Kc, Vc, dev(np.array([Lmax + 1000, 1 << 30], np.int32)), topk,
                                         scale, want_idx=True)
    torch.cuda.synchronize()
    assert int(idx.max()) < (Lmax - 1) // 64
    assert torch.equal(idx2, idx) and torch.equal(cnt2, cnt) and torch.equal(o2, o)

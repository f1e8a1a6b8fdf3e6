"""GPU parity of sas_pool_keys and sas_decode_select (long-context decode selection)
against the oracle's pool_keys / decode_block_scores / decode_select.

* Integer-valued keys and queries with a power-of-two scale make every pooled key and
  every score exact in bf16 / fp32 and in the oracle's float64, so pooled keys, scores,
  indices and counts are compared bit for bit; many scores tie, which exercises the
  lowest-index rule.
* N(0,1) inputs: pooled keys within one bf16 rounding of the float64 mean; scores within
  the bound that rounding implies (2^-8 scale sum_d |qbar_d kbar_d| plus fp32 slack);
  indices valid for the scores the kernel wrote (the K largest, lowest index on ties,
  ascending) and equal to the oracle's on every row whose K-th and (K+1)-th oracle scores
  are further apart than twice the score bound.
* Edge cases: no history (kv_len <= 64), one history block, budget 0 and above the
  history, partial last blocks, d = 64, G = 1, 5 and 8, first_block for incremental
  pooling, and the 512K-token context (C = 8191 history blocks) of the pages' longest
  decode measurement.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from learned_context_ranking_amd import sas, synth
from gpu_util import assert_close, dev, dev_bf16, host, log

pytestmark = pytest.mark.gpu


def _int_bits(shape, seed, lo=-2, hi=2):
    g = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits(g.integers(lo, hi + 1, size=shape).astype(np.float32))


def _pool_bound(ref):
    # one bf16 rounding (2^-9 relative) of an fp32 sum of 64 bf16 values
    return 2.0 ** -8 * np.abs(ref) + 1e-30


def test_pool_keys_normal_and_first_block():
    for d in (128, 64):
        log(f"pool_keys d={d}")
        B, Hkv, Lmax = 3, 2, 64 * 20
        kb = synth.normal_bf16((B, Hkv, Lmax, d), 4, synth.TID_K)
        kv_len = np.array([Lmax, 700, 63], np.int32)
        out = sas.sas_pool_keys(dev_bf16(kb), dev(kv_len))
        torch.cuda.synchronize()
        ref = oracle.pool_keys(synth.bf16_bits_to_f32(kb), kv_len)
        got = host(out)
        for b in range(B):
            full = kv_len[b] // 64
            assert np.all(np.abs(got[b, :, :full] - ref[b, :, :full]) <= _pool_bound(ref[b, :, :full]))
            assert np.all(got[b, :, full:] == 0.0)     # untouched (new tensor is zero)
        # incremental upkeep: only blocks >= first_block are written
        sentinel = torch.full((B, Hkv, Lmax // 64, d), 7.0, dtype=torch.bfloat16, device="cuda")
        sas.sas_pool_keys(dev_bf16(kb), dev(kv_len), first_block=5, out=sentinel)
        torch.cuda.synchronize()
        got2 = host(sentinel)
        assert np.all(got2[:, :, :5] == 7.0)
        for b in range(B):
            full = kv_len[b] // 64
            assert np.array_equal(got2[b, :, 5:full], got[b, :, 5:full])
            assert np.all(got2[b, :, max(full, 5):] == 7.0)


@pytest.mark.parametrize("Hq,Hkv,d,period", [(32, 8, 128, 0), (8, 8, 64, 0), (10, 2, 128, 7), (16, 2, 64, 5)])
def test_decode_select_exact_integer_inputs(Hq, Hkv, d, period):
    """Exact arithmetic on both sides: bit-identical pooled keys, scores, indices, counts,
    LSE within float rounding. With a period, the key blocks repeat every `period` blocks,
    so each row holds only that many distinct scores and the K-th is always tied."""
    log(f"decode_select exact Hq={Hq} Hkv={Hkv} d={d} period={period}")
    B, Lmax, topk = 4, 64 * 300, 16
    kb = _int_bits((B, Hkv, Lmax, d), Hq + d)
    if period:
        base = kb[:, :, :64 * period].reshape(B, Hkv, 1, 64 * period, d)
        reps = -(-Lmax // (64 * period))
        kb = np.ascontiguousarray(np.tile(base, (1, 1, reps, 1, 1)).reshape(B, Hkv, -1, d)[:, :, :Lmax])
    qb = _int_bits((B, Hq, d), Hq + d + 1)
    kv_len = np.array([Lmax, 64 * 17 + 1, 64, 64 * 123 + 40], np.int32)
    scale = 0.125
    K = dev_bf16(kb)
    kbar = sas.sas_pool_keys(K, dev(kv_len))
    s, idx, cnt, lse, logg = sas.sas_decode_select(dev_bf16(qb), kbar, dev(kv_len), scale, topk,
                                                   want_lse=True, want_logg=True)
    torch.cuda.synchronize()
    Kf = synth.bf16_bits_to_f32(kb)
    qf = synth.bf16_bits_to_f32(qb)
    assert np.array_equal(host(kbar), oracle.pool_keys(Kf, kv_len))
    s_r, idx_r, cnt_r, lse_r, logg_r = oracle.decode_select(qf, Kf, kv_len, scale, topk, kcap=topk)
    sg = host(s)
    hist = (kv_len - 1) // 64
    G = Hq // Hkv
    for b in range(B):
        if G & (G - 1) == 0:   # scale / G is a power of two: the scores themselves are exact
            assert np.array_equal(sg[b, :, :hist[b]], s_r[b, :, :hist[b]]), b
        else:                  # one fp32 rounding of scale / G; the order of the scores is exact
            np.testing.assert_allclose(sg[b, :, :hist[b]], s_r[b, :, :hist[b]], rtol=1e-6, atol=1e-7)
        assert np.all(np.isneginf(sg[b, :, hist[b]:]))
    assert np.array_equal(host(cnt), cnt_r)
    assert np.array_equal(host(idx), idx_r)
    fin = np.isfinite(lse_r)
    assert np.array_equal(np.isfinite(host(lse)), fin)
    np.testing.assert_allclose(host(lse)[fin], lse_r[fin], rtol=0, atol=1e-4)
    np.testing.assert_allclose(host(logg), logg_r, rtol=0, atol=1e-4)
    # many exact ties: the lowest-index rule decided some rows
    ties = sum(int(np.sum(s_r[b, h, :hist[b]] == s_r[b, h, idx_r[b, h, cnt_r[b, h] - 1]])) > 1
               for b in range(B) for h in range(Hkv) if cnt_r[b, h] > 0)
    assert ties > 0


def _check_valid_topk(s_row, n, topk, idx_row, cnt):
    """idx_row holds the min(topk, n) largest of s_row[:n] (NaN as -inf), ties to the lower
    index, ascending, -1 pad."""
    k = min(topk, n)
    assert cnt == k
    sel = idx_row[:k]
    assert np.all(idx_row[k:] == -1)
    assert np.all(np.diff(sel) > 0) and (k == 0 or (sel[0] >= 0 and sel[-1] < n))
    if k == 0 or k == n:
        return
    v = np.where(np.isnan(s_row[:n]), -np.inf, s_row[:n]).astype(np.float64)
    mask = np.zeros(n, bool); mask[sel] = True
    lo = v[mask].min()
    assert np.all(v[~mask] <= lo)
    # among blocks equal to the threshold, the kept ones come first
    eq_unsel = np.nonzero(~mask & (v == lo))[0]
    eq_sel = np.nonzero(mask & (v == lo))[0]
    if eq_unsel.size:
        assert eq_sel.max() < eq_unsel.min()


def _normal_case(B, Hq, Hkv, d, Lmax, kv_len, topk, seed, check_rows=None):
    log(f"decode_select normal B={B} Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} K={topk}")
    kb = synth.normal_bf16((B, Hkv, Lmax, d), seed, synth.TID_K)
    qb = synth.normal_bf16((B, Hq, 1, d), seed, synth.TID_QDEC)[:, :, 0]
    kv_len = np.asarray(kv_len, np.int32)
    scale = 1.0 / math.sqrt(d)
    kbar = sas.sas_pool_keys(dev_bf16(kb), dev(kv_len))
    s, idx, cnt, lse, _ = sas.sas_decode_select(dev_bf16(qb), kbar, dev(kv_len), scale, topk, want_lse=True)
    torch.cuda.synchronize()
    log("  GPU done; oracle")
    bs = list(range(B)) if check_rows is None else check_rows
    Kf = synth.bf16_bits_to_f32(kb[bs])
    qf = synth.bf16_bits_to_f32(qb[bs])
    kl = kv_len[bs]
    s_r, idx_r, cnt_r, lse_r, _ = oracle.decode_select(qf, Kf, kl, scale, topk, kcap=idx.shape[-1])
    kbar_r = oracle.pool_keys(Kf, kl)
    G = Hq // Hkv
    qbar = qf.astype(np.float64).reshape(len(bs), Hkv, G, d).mean(axis=2)
    sg, ig, cg, lg = host(s)[bs], host(idx)[bs], host(cnt)[bs], host(lse)[bs]
    exact_rows = 0
    for i in range(len(bs)):
        n = (kl[i] - 1) // 64
        for h in range(Hkv):
            bound = 2.0 ** -8 * scale * (np.abs(kbar_r[i, h, :n]) @ np.abs(qbar[i, h])) + 1e-5
            err = np.abs(sg[i, h, :n] - s_r[i, h, :n])
            assert np.all(err <= bound), (bs[i], h, float((err - bound).max()))
            _check_valid_topk(sg[i, h], n, topk, ig[i, h], cg[i, h])
            if 0 < topk < n:
                srt = np.sort(s_r[i, h, :n])[::-1]
                if srt[topk - 1] - srt[topk] > 2 * bound.max():
                    assert np.array_equal(ig[i, h], idx_r[i, h]), (bs[i], h)
                    exact_rows += 1
            if n > 0:
                assert abs(lg[i, h] - lse_r[i, h]) <= 1e-3 * max(1.0, abs(lse_r[i, h]))
            else:
                assert np.isneginf(lg[i, h])
    return exact_rows


def test_decode_select_normal_mixed_lengths():
    rows = _normal_case(6, 32, 8, 128, 64 * 512, [64 * 512, 64 * 300 + 7, 65, 64, 1, 64 * 2 + 1], 16, seed=2)
    log(f"  rows equal to the oracle's selection: {rows}")


@pytest.mark.parametrize("topk", [0, 1, 64, 600])
def test_decode_select_budgets(topk):
    _normal_case(2, 8, 2, 128, 64 * 400, [64 * 400, 64 * 150 + 3], topk, seed=5)


def test_decode_select_groups_and_small_d():
    _normal_case(3, 5, 1, 64, 64 * 257, [64 * 257, 64 * 256, 64 * 33], 8, seed=6)
    _normal_case(2, 16, 2, 64, 64 * 100, [6400, 3000], 4, seed=7)


def test_decode_select_planted_blocks_exact():
    """Keys of a few blocks aligned with the group's queries: those blocks rank first on both
    sides with wide margins, so the selection is compared exactly."""
    B, Hq, Hkv, d, Lmax, topk = 2, 8, 2, 128, 64 * 1000, 8
    g = np.random.default_rng(8)
    kf = 0.2 * g.standard_normal((B, Hkv, Lmax, d)).astype(np.float32)
    qf = g.standard_normal((B, Hq, d)).astype(np.float32)
    G = Hq // Hkv
    plant = {}
    for b in range(B):
        for h in range(Hkv):
            ms = np.sort(g.choice(999, size=topk, replace=False))
            plant[b, h] = ms
            u = qf[b, h * G:(h + 1) * G].mean(axis=0)
            for r, m in enumerate(ms):
                kf[b, h, m * 64:(m + 1) * 64] += (0.5 + 0.1 * r) * u / np.linalg.norm(u)
    kb = synth.f32_to_bf16_bits(kf)
    qb = synth.f32_to_bf16_bits(qf)
    kv_len = np.array([Lmax, Lmax], np.int32)
    kbar = sas.sas_pool_keys(dev_bf16(kb), dev(kv_len))
    _, idx, cnt, _, _ = sas.sas_decode_select(dev_bf16(qb), kbar, dev(kv_len), 1.0 / math.sqrt(d), topk)
    torch.cuda.synchronize()
    _, idx_r, cnt_r, _, _ = oracle.decode_select(synth.bf16_bits_to_f32(qb), synth.bf16_bits_to_f32(kb), kv_len,
                                                 1.0 / math.sqrt(d), topk)
    assert np.array_equal(host(idx), idx_r) and np.array_equal(host(cnt), cnt_r)
    for (b, h), ms in plant.items():
        assert np.array_equal(idx_r[b, h], ms)


def test_decode_select_then_decode_exact_inputs():
    """Selection feeds sas_decode on device; with exact selection the attention output
    matches the oracle's decode over the oracle's selection."""
    B, Hq, Hkv, d, Lmax, topk = 3, 8, 2, 128, 64 * 200, 16
    kb = _int_bits((B, Hkv, Lmax, d), 11)
    qb = _int_bits((B, Hq, d), 12)
    vb = synth.normal_bf16((B, Hkv, Lmax, d), 0, synth.TID_V)
    kv_len = np.array([Lmax, 64 * 77 + 5, 64 * 3], np.int32)
    scale = 0.125
    Kd, Qd = dev_bf16(kb), dev_bf16(qb)
    kbar = sas.sas_pool_keys(Kd, dev(kv_len))
    _, idx, cnt, _, _ = sas.sas_decode_select(Qd, kbar, dev(kv_len), scale, topk)
    o = sas.sas_decode(Qd, Kd, dev_bf16(vb), dev(kv_len), idx, cnt, scale)
    torch.cuda.synchronize()
    Kf, qf = synth.bf16_bits_to_f32(kb), synth.bf16_bits_to_f32(qb)
    _, idx_r, cnt_r, _, _ = oracle.decode_select(qf, Kf, kv_len, scale, topk)
    assert np.array_equal(host(idx), idx_r) and np.array_equal(host(cnt), cnt_r)
    ref = oracle.decode(qf, Kf, synth.bf16_bits_to_f32(vb), kv_len, idx_r, cnt_r, scale)
    assert_close("o", host(o), ref)


def test_decode_select_full_size_512k():
    """One sequence with a 512K-token cache (8,191 history blocks per KV head), 32 query /
    8 KV heads, d = 128, K = 16: every row checked."""
    _normal_case(1, 32, 8, 128, 64 * 8192, [64 * 8192], 16, seed=9)

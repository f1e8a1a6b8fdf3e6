"""Seeded synthetic inputs for SAS log-gated block-sparse attention.

This module holds random-number generation and dtype rounding only: no step of the
attention method lives here. Both the HIP path (through the tests and bench.py) and the
CPU oracle are fed from it, so it must stay free of the method's arithmetic.

Every tensor is drawn from ``numpy.random.default_rng([seed, tensor_id, chunk])`` where
``chunk`` enumerates the leading (batch, head) slices. A slice can therefore be
regenerated on its own, which is how the large-shape parity tests pick samples.

Tensor ids: Q=0, K=1, V=2, s=3, dO=4, plants/permutations=5, decode q=6.

Workload shapes come from the configurations the SAS pages train and serve at
(block 64, Top-K 32 at length 32,768, budgets of 1024-4096 tokens; the SAS summary page
on onedev.kr, sections "어떻게 쓰나" and "전제와 한계"). Head counts follow the Qwen3-4B
(32 query / 8 KV heads) and Qwen3-14B (40 / 8) attention shapes. No dataset item is used.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TID_Q, TID_K, TID_V, TID_S, TID_DO, TID_PLANT, TID_QDEC, TID_DG = 0, 1, 2, 3, 4, 5, 6, 7


def rng(seed: int, tensor_id: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tensor_id), int(chunk)])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; returns the raw uint16 bit patterns."""
    # Finite values and infinities cannot carry past bit 31 (NaN is patched below).
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    b = ((u + r) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        b[nan] = 0x7FC0
    return b


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, seed: int, tensor_id: int, threads: int | None = None) -> np.ndarray:
    """N(0,1) draws in fp32, rounded to bf16; returned as uint16 bit patterns.

    ``shape`` is (B, H, rows, d); one generator per (b, h) slice, so the result does not
    depend on how many threads fill it.
    """
    B, H = shape[0], shape[1]
    out = np.empty(shape, dtype=np.uint16)

    def fill(k):
        b, h = divmod(k, H)
        g = rng(seed, tensor_id, k)
        out[b, h] = f32_to_bf16_bits(g.standard_normal(shape[2:], dtype=np.float32))

    n = B * H
    threads = threads or min(16, os.cpu_count() or 1)
    if threads <= 1 or n <= 1:
        for k in range(n):
            fill(k)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(n)))
    return out


def normal_bf16_slice(shape, seed: int, tensor_id: int, b: int, h: int) -> np.ndarray:
    """One (b, h) slice of :func:`normal_bf16` without drawing the rest."""
    H = shape[1]
    g = rng(seed, tensor_id, b * H + h)
    return f32_to_bf16_bits(g.standard_normal(shape[2:], dtype=np.float32))


def scores_normal(shape, seed: int, mu: float = 0.0, sigma: float = 1.0) -> np.ndarray:
    """fp32 block scores ~ N(mu, sigma^2); ``shape`` = (B, H, rows, cols)."""
    B, H = shape[0], shape[1]
    out = np.empty(shape, dtype=np.float32)
    for b in range(B):
        for h in range(H):
            g = rng(seed, TID_S, b * H + h)
            out[b, h] = (mu + sigma * g.standard_normal(shape[2:], dtype=np.float32)).astype(np.float32)
    return out


def normal_f32(shape, seed: int, tensor_id: int, sigma: float = 1.0) -> np.ndarray:
    """fp32 N(0, sigma^2) draws of any shape from one generator (e.g. an upstream gradient)."""
    g = rng(seed, tensor_id)
    return (sigma * g.standard_normal(shape, dtype=np.float32)).astype(np.float32)


def scores_planted(B: int, H: int, NB: int, seed: int, nplant: int = 8,
                   mu: float = 4.0) -> np.ndarray:
    """N(0,1) background; for each (b, h, j) min(nplant, j) distinct history blocks m < j
    chosen uniformly are redrawn from N(mu, 1)."""
    s = scores_normal((B, H, NB, NB), seed)
    for b in range(B):
        for h in range(H):
            g = rng(seed, TID_PLANT, b * H + h)
            for j in range(1, NB):
                k = min(nplant, j)
                ms = g.choice(j, size=k, replace=False)
                s[b, h, j, ms] = (mu + g.standard_normal(k, dtype=np.float32)).astype(np.float32)
    return s


def scores_zipf(B: int, H: int, NB: int, seed: int, alpha: float = 1.1,
                sigma: float = 0.5) -> np.ndarray:
    """One random ranking of block ids per (b, h), shared by every query block:
    s[j, m] = -alpha * ln(rank(m)) + N(0, sigma^2) with rank in 1..NB."""
    out = np.empty((B, H, NB, NB), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            g = rng(seed, TID_PLANT, b * H + h)
            perm = g.permutation(NB)
            rank = np.empty(NB, dtype=np.float64)
            rank[perm] = np.arange(1, NB + 1)
            base = (-alpha * np.log(rank)).astype(np.float32)
            gn = rng(seed, TID_S, b * H + h)
            out[b, h] = (base[None, :] + sigma * gn.standard_normal((NB, NB), dtype=np.float32)).astype(np.float32)
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    n: int            # tokens per sequence (prefill) or KV length (decode)
    topk: int
    block: int = 64
    scores: str = "normal"   # normal | planted | zipf
    decode: bool = False
    backward: bool = True
    seed: int = 0

    @property
    def NB(self) -> int:
        return self.n // self.block

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 64, 1024, 4),
    "qwen3_4b_train": Workload("qwen3_4b_train", 1, 32, 8, 128, 32768, 32),
    "decode": Workload("decode", 64, 32, 8, 128, 32768, 16, decode=True, backward=False),
    "long_prefill": Workload("long_prefill", 1, 32, 8, 128, 131072, 64, scores="planted",
                             backward=False),
    "qwen3_14b_k16": Workload("qwen3_14b_k16", 1, 40, 8, 128, 32768, 16, scores="zipf"),
    "qwen3_14b_k32": Workload("qwen3_14b_k32", 1, 40, 8, 128, 32768, 32, scores="zipf"),
    "qwen3_14b_k64": Workload("qwen3_14b_k64", 1, 40, 8, 128, 32768, 64, scores="zipf"),
}


def prefill_scores(w: Workload) -> np.ndarray:
    if w.scores == "normal":
        return scores_normal((w.B, w.Hkv, w.NB, w.NB), w.seed)
    if w.scores == "planted":
        return scores_planted(w.B, w.Hkv, w.NB, w.seed)
    if w.scores == "zipf":
        return scores_zipf(w.B, w.Hkv, w.NB, w.seed)
    raise ValueError(w.scores)

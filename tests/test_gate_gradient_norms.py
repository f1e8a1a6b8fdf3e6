"""Score-gradient norms under the method's gate (softmax over every history block) and the
kept-set normalisation a binary Top-K mask implies ([SAS-ko] "무엇과 다른가", choice 3: the
explainer reports that the kept-set normalisation makes the gradient norm much larger than
soft gating at a random-init selector). Through the oracle's chain select -> forward ->
backward (dg) -> score gradient, on near-uniform scores (a random-init selector, N(0, 0.02))
and N(0,1) tensors. This reports a quantity; it is not a parity pin.

On these synthetic inputs the kept-set normalisation gives the larger norm, and the gap
widens as the history grows against the budget; it stays a small factor (about 1.3x here)
rather than the explainer's tens of times, which it reports for a real model's loss:
with random upstream gradients dg has random signs, so the normalisation term stays small.
"""
import math

import numpy as np

import oracle
from learned_context_ranking_amd import synth


def _ds_norms(NB, K, sigma=0.02, d=64):
    n = NB * 64
    f = synth.bf16_bits_to_f32
    q = f(synth.normal_bf16((1, 1, n, d), 0, synth.TID_Q))
    k = f(synth.normal_bf16((1, 1, n, d), 0, synth.TID_K))
    v = f(synth.normal_bf16((1, 1, n, d), 0, synth.TID_V))
    do = f(synth.normal_bf16((1, 1, n, d), 0, synth.TID_DO))
    s = synth.scores_normal((1, 1, NB, NB), 0, sigma=sigma)
    out = {}
    for gate in ("softmax", "softmax_selected"):
        idx, cnt, _, logg = oracle.select_prefill(s, K, gate=gate)
        _, _, _, dg = oracle.attn_bwd(q, k, v, do, idx, cnt, logg, 1.0 / math.sqrt(d))
        ds = oracle.gates_bwd_prefill(s, idx, cnt, dg, gate=gate)
        out[gate] = float(np.linalg.norm(ds))
    return out


def test_kept_set_normalisation_gives_larger_score_gradients():
    ratios = []
    for NB, K in ((32, 4), (64, 4)):
        n = _ds_norms(NB, K)
        r = n["softmax_selected"] / n["softmax"]
        print(f"NB={NB} K={K}: |ds| softmax {n['softmax']:.3f}, kept-set softmax "
              f"{n['softmax_selected']:.3f}, ratio {r:.3f}")
        ratios.append(r)
        assert r > 1.0
    assert ratios[1] > ratios[0]   # longer history against the same budget: larger gap

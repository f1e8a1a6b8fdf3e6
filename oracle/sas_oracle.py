"""Oracle: a plain, slow CPU implementation of SAS log-gated block-sparse attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(``learned_context_ranking_amd``) never imports it, and this module imports nothing
from the product: the two share only the seeded input generator, which carries none of
the method's arithmetic.

Everything here is NumPy in float64, applied to inputs that are exactly representable
(bf16-rounded draws, fp32 scores), one query block at a time, with a matrix product as
the only library step. It follows the pages' notation: block size ``b``, history blocks
``m < j`` of query block ``j``, scores ``s``, gates ``g = softmax(s)`` with the current
block's gate fixed at 1, the Top-K set ``I`` and the key set ``S = B_j U (U_{m in I} B_m)``.

Sources, cited by page title and section:

* [SAS-ja] "論文解説: SAS — 疎注意の「どのブロックを読むか」を言語モデル損失で端から端まで学習する"
  (ta-paperlens.web.app). Section "前提" restates the paper's section 3 (n tokens in
  C = n/b blocks, selector scores s in R^C, the Top-K union S, per-query cost |S|).
  Section "仕組み" restates section 4.1 (positive gates g = phi(s), current block gate 1,
  one gate per block broadcast to its tokens), section 4.3 eq. (9) (log g added to the
  logits inside the softmax; exp(z + log g) = g exp(z)) and Algorithm 2 / section 5.1
  (inference: Top-K on s, no gates, plain sparse attention).
* [PBS-ja] "Sparser Block-Sparse Attention via Token Permutation" (gist.science/ja/paper/
  2510.21270), prior art cited for one step only: sections "3." (proxy scoring) and
  "4. 実装" (block selection) estimate a block's importance by mean pooling of attention
  scores, which stands in for the undefined SAS selector in long-context decode selection.
* [S2O-ja] "S2O: オンライン置換によるスパースアテンションの早期停止" summary (gist.science/ja/paper/
  2602.22575), prior art cited for one rule only: section "2. 早期停止ルール" stops adding
  blocks, taken in descending importance, once a block's marginal softmax mass falls
  below a threshold relative to the mass accumulated so far.
* [SAS-ko] "SAS는 언어모델 손실로 문맥 순위를 직접 학습하는 사후 어텐션 희소화다"
  (onedev.kr/papers/5). Section "어떻게 동작하나" gives o = softmax(q K_S^T + log g_S) V_S.
  Section "무엇과 다른가" gives the four design choices: (1) the gate inside the softmax and
  its gradient dg_m = sum_{i in B_m} (p~_i / g_m) dO^T (v_i - o); (2) g = softmax(s), so
  log g_m = s_m - LSE(s), invariant to a global shift of s; (4) sparse training scope.

Readings taken where the pages are silent (each also stated where it is used):

* R1 scale: logits are ``scale * q.k`` (the pages drop the scale); ``log g`` is added
  unscaled so that exp(z + log g) = g exp(z) holds exactly.
* R2 the gate softmax normalises over every valid history block m < j of the row, not
  only the selected ones.
* R3 s, I and g are shared by the b queries of a query block and by the G query heads
  of a KV head; dg sums over those G*b rows.
* R4 query block j sees history blocks 0..j-1 and its own block with a causal mask.
* R5 ties in s go to the lowest block index; -0 equals +0; NaN ranks as -inf.
* R6 selected indices are reported in ascending order, padded with -1 (logg with 0).
* R7 decode: the query is the last of kv_len tokens; its current block holds tokens
  [b*floor((L-1)/b), L); history is the blocks before it; attention is ungated unless
  log-gates are supplied.
* R8 dg is the derivative with respect to g itself, reported per selected slot.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------- gates and selection

def _rank_keys(s_row):
    """Scores as the selection compares them (R5): NaN -> -inf, -0 -> +0."""
    s = np.array(s_row, dtype=np.float64)
    s[np.isnan(s)] = NEG_INF
    s[s == 0.0] = 0.0
    return s


def row_log_gates(s_row):
    """Log-gates of one row of history scores.

    [SAS-ko] "무엇과 다른가", choice 2: g = softmax(s), so log g_m = s_m - LSE(s).
    [SAS-ja] "仕組み": the current block's gate is 1 (log-gate 0) and is not part of s.
    Returns (LSE, log g) with LSE = -inf and an empty vector for a row with no history.
    A NaN score is read as -inf (R5), so its gate is 0.
    """
    s = _rank_keys(s_row)
    if s.size == 0:
        return NEG_INF, s
    mx = s.max()
    if mx == NEG_INF:
        return NEG_INF, np.full_like(s, NEG_INF)
    lse = mx + np.log(np.sum(np.exp(s - mx)))
    return lse, s - lse


GATES = ("softmax", "softmax_selected", "sigmoid", "exp")


def row_log_gates_variant(s_row, sel, gate):
    """Log-gates of the selected blocks ``sel`` of one row under a gate activation phi
    ([SAS-ko] "무엇과 다른가", choices 2 and 3 and the alternatives they are compared with):

    * "softmax": g = softmax(s) over every valid history block (choice 2; row_log_gates);
    * "softmax_selected": g = softmax(s) over the selected set only, the normalisation a
      binary Top-K mask trained with a straight-through estimator implies (choice 3);
    * "sigmoid": g = sigmoid(s), log g = -log(1 + exp(-s));
    * "exp": the raw score injected as the logit, log g = s (unnormalised).
    Returns (normaliser, log g[sel]): LSE over the valid blocks, LSE over the selected
    ones, or 0 for the unnormalised gates. NaN scores read as -inf (gate 0).
    """
    s = _rank_keys(s_row)
    sel = np.asarray(sel, dtype=np.int64)
    if gate == "softmax":
        lse, lg = row_log_gates(s_row)
        return lse, lg[sel]
    x = s[sel]
    if gate == "softmax_selected":
        if x.size == 0 or x.max() == NEG_INF:
            return NEG_INF, np.full_like(x, NEG_INF)
        mx = x.max()
        lse = mx + np.log(np.sum(np.exp(x - mx)))
        return lse, x - lse
    if gate == "sigmoid":
        # log sigmoid(x) = -log(1 + e^-x), evaluated without overflow on either side
        return 0.0, np.where(x >= 0, -np.log1p(np.exp(-np.abs(x))), x - np.log1p(np.exp(-np.abs(x))))
    if gate == "exp":
        return 0.0, x.copy()
    raise ValueError(f"unknown gate {gate!r}")


def row_topk(s_row, k):
    """The k highest-scoring history blocks of one row, ties to the lowest index (R5),
    reported in ascending block order (R6).

    [SAS-ja] "前提": the selector's Top-K blocks form the attended set.
    """
    s = _rank_keys(s_row)
    k = min(int(k), s.size)
    order = np.lexsort((np.arange(s.size), -s))   # primary key -s, then the block index
    return np.sort(order[:k])


def select(s, valid, topk, full_scope=False, kcap=None, gate="softmax"):
    """Gates plus Top-K selection for a stack of score rows.

    s: [R, ld] fp32 scores; row r has ``valid[r]`` history blocks (columns 0..valid-1).
    Sparse scope keeps min(topk, valid) blocks; full scope keeps all of them
    ([SAS-ko] "무엇과 다른가", choice 4). ``gate`` picks phi (row_log_gates_variant).
    Returns idx [R, kcap] int32 (ascending, -1 pad), cnt [R] int32, lse [R] float64 (the
    gate's normaliser), logg [R, kcap] float64 (log g of each selected block, 0 pad).
    """
    s = np.asarray(s)
    R = s.shape[0]
    valid = np.broadcast_to(np.asarray(valid, dtype=np.int64), (R,))
    if kcap is None:
        kcap = int(valid.max()) if full_scope else int(topk)
    idx = np.full((R, kcap), -1, dtype=np.int32)
    cnt = np.zeros(R, dtype=np.int32)
    lse = np.full(R, NEG_INF, dtype=np.float64)
    logg = np.zeros((R, kcap), dtype=np.float64)
    for r in range(R):
        row = s[r, : valid[r]]
        k = row.size if full_scope else min(int(topk), row.size)
        if k > kcap:
            raise ValueError("kcap smaller than the number of selected blocks")
        sel = row_topk(row, k)
        idx[r, :k] = sel
        cnt[r] = k
        lse[r], logg[r, :k] = row_log_gates_variant(row, sel, gate)
    return idx, cnt, lse, logg


def select_prefill(s, topk, full_scope=False, kcap=None, gate="softmax"):
    """Selection for prefill/training score tensors s [B, H, NB, NB]: row j has j valid
    history blocks (R4). Returns tensors shaped [B, H, NB, kcap] / [B, H, NB]."""
    B, H, NB, ld = s.shape
    valid = np.tile(np.arange(NB), B * H)
    idx, cnt, lse, logg = select(s.reshape(B * H * NB, ld), valid, topk, full_scope, kcap, gate)
    kc = idx.shape[1]
    return (idx.reshape(B, H, NB, kc), cnt.reshape(B, H, NB), lse.reshape(B, H, NB),
            logg.reshape(B, H, NB, kc))


def gates_bwd(s, valid, idx, cnt, dg, gate="softmax"):
    """Gradient with respect to the scores through the gate activation.

    [SAS-ko] "무엇과 다른가", choice 2: g = softmax(s) over the row's valid history blocks
    (R2). dg holds dL/dg for the selected blocks, aligned with idx (R8); an unselected block
    has no gradient of its own (choice 4, sparse scope), so its entry of dL/dg is 0. The
    chain rule through the softmax, whose Jacobian is diag(g) - g g^T, gives
    ds_m = g_m (dg_m - sum_m' g_m' dg_m') for every valid m. A NaN or -inf score has g = 0
    (R5), hence ds = 0. Entries m >= valid are 0.
    The other activations of row_log_gates_variant: "softmax_selected" applies the same
    Jacobian over the selected set only (ds = 0 elsewhere); "sigmoid" gives
    ds_m = dg_m g_m (1 - g_m) and "exp" ds_m = dg_m g_m, on the selected blocks.
    s: [R, ld]; valid [R]; idx, dg [R, kcap]; cnt [R]. Returns ds [R, ld] float64.
    """
    s = np.asarray(s)
    R, ld = s.shape
    valid = np.broadcast_to(np.asarray(valid, dtype=np.int64), (R,))
    ds = np.zeros((R, ld), dtype=np.float64)
    for r in range(R):
        v = int(valid[r])
        if v == 0:
            continue
        c = int(cnt[r])
        sel = np.asarray(idx[r, :c], dtype=np.int64)
        dgs = np.asarray(dg[r, :c], dtype=np.float64)
        if gate == "softmax":
            _, lg = row_log_gates(s[r, :v])
            g = np.exp(lg)
            dgf = np.zeros(v)
            dgf[sel] = dgs
            ds[r, :v] = g * dgf - g * np.dot(g, dgf)
            continue
        _, lg = row_log_gates_variant(s[r, :v], sel, gate)
        g = np.exp(lg)
        if gate == "softmax_selected":
            ds[r, sel] = g * dgs - g * np.dot(g, dgs)
        elif gate == "sigmoid":
            ds[r, sel] = dgs * g * (1.0 - g)
        elif gate == "exp":
            ds[r, sel] = dgs * g
        else:
            raise ValueError(f"unknown gate {gate!r}")
    return ds


def gates_bwd_prefill(s, idx, cnt, dg, gate="softmax"):
    """gates_bwd for prefill score tensors s [B, H, NB, NB] (row j has j valid blocks)."""
    B, H, NB, ld = s.shape
    valid = np.tile(np.arange(NB), B * H)
    kc = idx.shape[-1]
    R = B * H * NB
    ds = gates_bwd(s.reshape(R, ld), valid, idx.reshape(R, kc), cnt.reshape(R), dg.reshape(R, kc), gate)
    return ds.reshape(B, H, NB, ld)


# ---------------------------------------------------------------- training forward/backward

def _key_set(j, idx_row, cnt_j, logg_row, block):
    """Token indices of S_j = B_j U (U_{m in I_j} B_m) and the additive log-gate of each
    ([SAS-ja] "仕組み": each block's gate is broadcast to all of its tokens; the current
    block's gate is 1)."""
    toks = [np.arange(j * block, (j + 1) * block)]
    ell = [np.zeros(block)]
    for t in range(int(cnt_j)):
        m = int(idx_row[t])
        toks.append(np.arange(m * block, (m + 1) * block))
        ell.append(np.full(block, float(logg_row[t])))
    return np.concatenate(toks), np.concatenate(ell)


def _block_logits(q, Kb, keys, ell, j, block, scale):
    """Logits of one query block over S_j: z_ti = scale * q_t.k_i + log g_{m(i)}
    ([SAS-ko] "어떻게 동작하나": softmax(q K_S^T + log g_S); R1), -inf above the diagonal
    of the current block (R4). Returns (z, zu) where zu is z before the gate is added."""
    zu = scale * (q @ Kb.T)
    qpos = j * block + np.arange(q.shape[0])
    zu = np.where(keys[None, :] > qpos[:, None], NEG_INF, zu)
    return zu + ell[None, :], zu


def fwd_query_block(Q, K, V, b, h, j, idx_row, cnt_j, logg_row, scale, block=64, placement="inside"):
    """One query block of the forward for every query head of KV head h: returns
    O [G, block, d] and LSE [G, block] (eq. (9) of [SAS-ja] "仕組み").

    placement "outside" is the alternative of [SAS-ko] "무엇과 다른가", choice 1: the gate
    multiplies the attention probabilities after the softmax, o = sum_i p_i g_m(i) v_i with
    p = softmax(scale q K_S^T) (no gate in the logits); LSE is then that of the ungated
    logits."""
    Hq, Hkv = Q.shape[1], K.shape[1]
    G = Hq // Hkv
    keys, ell = _key_set(j, idx_row, cnt_j, logg_row, block)
    Kb = np.asarray(K[b, h, keys], np.float64)
    Vb = np.asarray(V[b, h, keys], np.float64)
    rows = slice(j * block, (j + 1) * block)
    O = np.zeros((G, block, Q.shape[-1]))
    LSE = np.zeros((G, block))
    for g in range(G):
        q = np.asarray(Q[b, h * G + g, rows], np.float64)
        z, zu = _block_logits(q, Kb, keys, ell, j, block, scale)
        if placement == "outside":
            mx = zu.max(axis=1, keepdims=True)
            e = np.exp(zu - mx)
            Z = e.sum(axis=1, keepdims=True)
            O[g] = ((e / Z) * np.exp(ell)[None, :]) @ Vb
        else:
            mx = z.max(axis=1, keepdims=True)
            e = np.exp(z - mx)
            Z = e.sum(axis=1, keepdims=True)
            O[g] = (e / Z) @ Vb
        LSE[g] = (mx + np.log(Z))[:, 0]
    return O, LSE


def attn_fwd(Q, K, V, idx, cnt, logg, scale, block=64, placement="inside"):
    """Gated block-sparse attention forward, eq. (9) of [SAS-ja] "仕組み".

    Q [B, Hq, n, d]; K, V [B, Hkv, n, d]; idx/logg [B, Hkv, NB, kcap]; cnt [B, Hkv, NB].
    Returns O [B, Hq, n, d] and the natural-log row sums LSE [B, Hq, n].
    """
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    NB = n // block
    O = np.zeros((B, Hq, n, d))
    LSE = np.zeros((B, Hq, n))
    for b in range(B):
        for h in range(Hkv):
            for j in range(NB):
                o, l = fwd_query_block(Q, K, V, b, h, j, idx[b, h, j], cnt[b, h, j], logg[b, h, j],
                                       scale, block, placement)
                rows = slice(j * block, (j + 1) * block)
                O[b, h * G:(h + 1) * G, rows] = o
                LSE[b, h * G:(h + 1) * G, rows] = l
    return O, LSE


def bwd_query_block(Q, K, V, dO, b, h, j, idx_row, cnt_j, logg_row, scale, block=64, placement="inside"):
    """Backward contributions of one query block (all G query heads of KV head h).

    Content gradients are those of softmax attention over S_j; gradients reach only the
    attended keys (sparse scope, [SAS-ko] "무엇과 다른가", choice 4). The gate gradient of
    selected block m follows choice 1 of the same section:
    dg_jm = sum over the G*b query rows t of the group (R3) and keys i in B_m of
    (p~_ti / g_jm) * dO_t^T (v_i - o_t). By eq. (9) p~_ti / g_jm = exp(z_ti - LSE_t) with
    z_ti the logit before the gate is added, which is what is evaluated (it stays
    defined when g_jm = 0).
    With placement "outside" (choice 1's alternative, see fwd_query_block) the weights are
    w_ti = p_ti g_m(i): dV = w^T dO, the probabilities' gradient is g_m(i) dO_t^T v_i,
    dS = p (g dP - delta) with the same delta = dO_t^T o_t, and the gate gradient is the
    one the explainer gives for that placement, dg_jm = sum_{t, i in B_m} p_ti dO_t^T v_i.
    Returns dQ [G, block, d], the key token indices of S_j, dK and dV over those keys
    ([len(keys), d], summed over the G heads) and dg [cnt_j].
    """
    Hq, Hkv = Q.shape[1], K.shape[1]
    G = Hq // Hkv
    keys, ell = _key_set(j, idx_row, cnt_j, logg_row, block)
    Kb = np.asarray(K[b, h, keys], np.float64)
    Vb = np.asarray(V[b, h, keys], np.float64)
    rows = slice(j * block, (j + 1) * block)
    d = Q.shape[-1]
    dQ = np.zeros((G, block, d))
    dKs = np.zeros((len(keys), d))
    dVs = np.zeros((len(keys), d))
    dg = np.zeros(int(cnt_j))
    for g in range(G):
        q = np.asarray(Q[b, h * G + g, rows], np.float64)
        z, zu = _block_logits(q, Kb, keys, ell, j, block, scale)
        if placement == "outside":
            mx = zu.max(axis=1, keepdims=True)
            e = np.exp(zu - mx)
            P = e / e.sum(axis=1, keepdims=True)
            gk = np.exp(ell)[None, :]                    # gate of each key's block
            W = P * gk
            o = W @ Vb
            do = np.asarray(dO[b, h * G + g, rows], np.float64)
            dP = do @ Vb.T
            delta = np.sum(do * o, axis=1, keepdims=True)
            dS = P * (gk * dP - delta)
            dQ[g] = scale * (dS @ Kb)
            dKs += scale * (dS.T @ q)
            dVs += W.T @ do
            for t in range(int(cnt_j)):
                cols = slice(block * (t + 1), block * (t + 2))
                dg[t] += np.sum(P[:, cols] * dP[:, cols])
            continue
        mx = z.max(axis=1, keepdims=True)
        e = np.exp(z - mx)
        Z = e.sum(axis=1, keepdims=True)
        P = e / Z
        lse = mx + np.log(Z)
        o = P @ Vb
        do = np.asarray(dO[b, h * G + g, rows], np.float64)
        dP = do @ Vb.T                                   # dO_t^T v_i
        delta = np.sum(do * o, axis=1, keepdims=True)    # dO_t^T o_t
        dS = P * (dP - delta)
        dQ[g] = scale * (dS @ Kb)
        dKs += scale * (dS.T @ q)
        dVs += P.T @ do
        ratio = np.exp(zu - lse)                         # = p~ / g
        for t in range(int(cnt_j)):
            cols = slice(block * (t + 1), block * (t + 2))
            dg[t] += np.sum(ratio[:, cols] * (dP[:, cols] - delta))
    return dQ, keys, dKs, dVs, dg


def attn_bwd(Q, K, V, dO, idx, cnt, logg, scale, block=64, placement="inside"):
    """Backward of :func:`attn_fwd` with the gate gradient (see :func:`bwd_query_block`).
    Returns dQ, dK, dV (float64, shapes of Q, K, V) and dg [B, Hkv, NB, kcap] (0 pad)."""
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    NB = n // block
    kcap = idx.shape[-1]
    dQ = np.zeros((B, Hq, n, d)); dK = np.zeros((B, Hkv, n, d)); dV = np.zeros((B, Hkv, n, d))
    dg = np.zeros((B, Hkv, NB, kcap))
    for b in range(B):
        for h in range(Hkv):
            for j in range(NB):
                c = int(cnt[b, h, j])
                dq, keys, dks, dvs, dgj = bwd_query_block(Q, K, V, dO, b, h, j, idx[b, h, j], c,
                                                          logg[b, h, j], scale, block, placement)
                dQ[b, h * G:(h + 1) * G, j * block:(j + 1) * block] = dq
                np.add.at(dK[b, h], keys, dks)
                np.add.at(dV[b, h], keys, dvs)
                dg[b, h, j, :c] = dgj
    return dQ, dK, dV, dg


def dense_causal(Q, K, V, scale):
    """Ordinary causal softmax attention over every earlier token ([SAS-ja] "前提": the
    dense attention the sparse form replaces). Used to pin the full-scope, ungated case."""
    Q = np.asarray(Q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
    B, Hq, n, d = Q.shape
    G = Hq // K.shape[1]
    O = np.zeros_like(Q)
    mask = np.triu(np.ones((n, n), dtype=bool), 1)
    for b in range(B):
        for hq in range(Hq):
            z = scale * Q[b, hq] @ K[b, hq // G].T
            z[mask] = NEG_INF
            e = np.exp(z - z.max(axis=1, keepdims=True))
            O[b, hq] = (e / e.sum(axis=1, keepdims=True)) @ V[b, hq // G]
    return O


# ---------------------------------------------------------------- decode (Algorithm 2)

def decode_rows_valid(kv_len, block=64):
    """History blocks of each decode sequence: the blocks before the one holding token
    kv_len - 1 (R7)."""
    return (np.asarray(kv_len, dtype=np.int64) - 1) // block


def decode(q, Kc, Vc, kv_len, idx, cnt, scale, block=64, logg=None):
    """Inference form, [SAS-ja] "仕組み", Algorithm 2 / section 5.1: Top-K on s, then plain
    (ungated) sparse attention over the current block plus the selected blocks.

    q [B, Hq, d]; Kc, Vc [B, Hkv, Lmax, d]; kv_len [B]; idx [B, Hkv, kcap]; cnt [B, Hkv].
    With ``logg`` ([B, Hkv, kcap]) the log-gates are added as in training (a check only).
    Returns o [B, Hq, d].
    """
    q = np.asarray(q, np.float64); Kc = np.asarray(Kc, np.float64); Vc = np.asarray(Vc, np.float64)
    B, Hq, d = q.shape
    Hkv = Kc.shape[1]
    G = Hq // Hkv
    o = np.zeros_like(q)
    for b in range(B):
        L = int(kv_len[b])
        c = (L - 1) // block
        for h in range(Hkv):
            toks = [np.arange(c * block, L)]
            ell = [np.zeros(L - c * block)]
            for t in range(int(cnt[b, h])):
                m = int(idx[b, h, t])
                toks.append(np.arange(m * block, (m + 1) * block))
                ell.append(np.full(block, 0.0 if logg is None else float(logg[b, h, t])))
            keys = np.concatenate(toks)
            ell = np.concatenate(ell)
            Kb, Vb = Kc[b, h, keys], Vc[b, h, keys]
            for g in range(G):
                z = scale * (Kb @ q[b, h * G + g]) + ell
                e = np.exp(z - z.max())
                o[b, h * G + g] = (e / e.sum()) @ Vb
    return o


# ---------------------------------------------------------------- long-context decode selection

def pool_keys(Kc, kv_len, block=64):
    """Block means of the key cache: kbar[b, h, m] = (1/b) sum_{i in B_m} k_i for every
    complete block m ((m + 1) * b <= kv_len[b]); incomplete and absent blocks are 0.

    A cache of these means turns the block score below into one dot product per block.
    Kc [B, Hkv, Lmax, d]; returns [B, Hkv, Lmax // b, d] float64.
    """
    Kc = np.asarray(Kc, np.float64)
    B, Hkv, Lmax, d = Kc.shape
    C = Lmax // block
    out = np.zeros((B, Hkv, C, d))
    for b in range(B):
        full = min(int(kv_len[b]) // block, C)
        if full > 0:
            out[b, :, :full] = Kc[b, :, :full * block].reshape(Hkv, full, block, d).mean(axis=2)
    return out


def decode_block_scores(q, Kc, kv_len, scale, block=64):
    """Stand-in selector score of each history block for one decode step.

    The pages do not define the selector network (AttnGate), so block importance is taken
    as in [PBS-ja] "4. 実装" (block selection) and "3." (proxy scoring): the mean of the
    attention scores over the block. Here the mean runs over the b keys of block m and the
    G query heads of the KV group (one score row per (sequence, KV head), R3):
    s[b, h, m] = mean_{g, i in B_m} scale * q_{hG+g} . k_i, for the history blocks
    m < (kv_len - 1) // b (R7); later entries are -inf.
    q [B, Hq, d]; Kc [B, Hkv, Lmax, d]; returns [B, Hkv, Lmax // b] float64.
    """
    q = np.asarray(q, np.float64)
    Kc = np.asarray(Kc, np.float64)
    B, Hq, d = q.shape
    Hkv, Lmax = Kc.shape[1], Kc.shape[2]
    G = Hq // Hkv
    C = Lmax // block
    s = np.full((B, Hkv, C), NEG_INF)
    for b in range(B):
        hist = int(decode_rows_valid(kv_len[b], block))
        if hist <= 0:
            continue
        for h in range(Hkv):
            logits = scale * (q[b, h * G:(h + 1) * G] @ Kc[b, h, :hist * block].T)   # [G, hist * b]
            s[b, h, :hist] = logits.reshape(G, hist, block).mean(axis=(0, 2))
    return s


def decode_select(q, Kc, kv_len, scale, topk, kcap=None, block=64):
    """Block scores plus Top-K for one decode step (Algorithm 2 of [SAS-ja] "仕組み":
    the K best-scoring history blocks). Returns (s, idx [B, Hkv, kcap], cnt [B, Hkv],
    lse [B, Hkv], logg [B, Hkv, kcap])."""
    s = decode_block_scores(q, Kc, kv_len, scale, block)
    B, Hkv, C = s.shape
    valid = np.repeat(decode_rows_valid(kv_len, block), Hkv)
    idx, cnt, lse, logg = select(s.reshape(B * Hkv, C), valid, topk, kcap=kcap)
    kc = idx.shape[-1]
    return s, idx.reshape(B, Hkv, kc), cnt.reshape(B, Hkv), lse.reshape(B, Hkv), logg.reshape(B, Hkv, kc)


# ---------------------------------------------------------------- paged decode

def gather_pages(pool, page_table, kv_len, block=64):
    """The logical cache of each sequence from a paged pool: pool [P, Hkv, b, d] holds
    one block of b tokens per page; page_table[b, m] is the page of logical block m.
    Returns [B, Hkv, Lmax, d] with Lmax = page_table.shape[1] * b; blocks at or past
    ceil(kv_len / b) are zero."""
    pool = np.asarray(pool, np.float64)
    B, maxp = page_table.shape
    Hkv, d = pool.shape[1], pool.shape[3]
    out = np.zeros((B, Hkv, maxp * block, d))
    for b in range(B):
        for m in range(-(-int(kv_len[b]) // block)):
            out[b, :, m * block:(m + 1) * block] = pool[int(page_table[b, m])]
    return out


def decode_paged(q, Kpool, Vpool, page_table, kv_len, idx, cnt, scale, block=64, logg=None):
    """Decode (Algorithm 2 of [SAS-ja] "仕組み") over a paged cache: the same attention as
    ``decode`` on the logical cache the page table describes."""
    Kc = gather_pages(Kpool, page_table, kv_len, block)
    Vc = gather_pages(Vpool, page_table, kv_len, block)
    return decode(q, Kc, Vc, kv_len, idx, cnt, scale, block, logg)


# ---------------------------------------------------------------- early-stopped decode

def decode_early_stop(q, Kc, Vc, kv_len, idx, cnt, order, scale, tau, block=64):
    """Decode with a mass-threshold early stop over the selected blocks, the stopping rule
    of [S2O-ja] (gist.science/ja/paper/2602.22575), section "2. 早期停止ルール", and the
    two-pass order of its section "3. カーネル実装" (prior art, used as a budget rule):

    per query head, the online-softmax state starts from the current block (causal, as in
    decode); the selected blocks then follow in descending ``order`` (ties to the lower
    block index). Each block's marginal softmax mass dl = sum_i exp(z_i - M) is compared
    with the mass l accumulated before it (both in the frame of the running maximum M
    after the block): the block is added, and if dl < tau * l the remaining blocks are
    skipped. tau = 0 never stops early (plain decode over every selected block).

    q [B, Hq, d]; Kc, Vc [B, Hkv, Lmax, d]; idx, order [B, Hkv, kcap]; cnt [B, Hkv].
    Returns (o [B, Hq, d], used [B, Hq]: history blocks each head attended,
    margin: the smallest |dl / l - tau| over the comparisons made, relative to tau).
    """
    q = np.asarray(q, np.float64); Kc = np.asarray(Kc, np.float64); Vc = np.asarray(Vc, np.float64)
    B, Hq, d = q.shape
    Hkv = Kc.shape[1]
    G = Hq // Hkv
    o = np.zeros_like(q)
    used = np.zeros((B, Hq), dtype=np.int32)
    margin = np.inf
    for b in range(B):
        L = int(kv_len[b])
        c = (L - 1) // block
        for h in range(Hkv):
            k = int(cnt[b, h])
            sel = np.asarray(idx[b, h, :k], dtype=np.int64)
            key = np.asarray(order[b, h, :k], dtype=np.float64)
            seq = sel[np.lexsort((sel, -key))]          # descending order, ties to the lower index
            for g in range(G):
                qv = q[b, h * G + g]
                z = scale * (Kc[b, h, c * block:L] @ qv)
                M = z.max()
                w = np.exp(z - M)
                l = w.sum()
                acc = w @ Vc[b, h, c * block:L]
                n_used = 0
                for m in seq:
                    zb = scale * (Kc[b, h, m * block:(m + 1) * block] @ qv)
                    Mn = max(M, zb.max())
                    l *= np.exp(M - Mn)
                    acc *= np.exp(M - Mn)
                    M = Mn
                    wb = np.exp(zb - M)
                    dl = wb.sum()
                    stop = dl < tau * l
                    if tau > 0:
                        margin = min(margin, abs(dl / l - tau) / tau)
                    l += dl
                    acc += wb @ Vc[b, h, m * block:(m + 1) * block]
                    n_used += 1
                    if stop:
                        break
                o[b, h * G + g] = acc / l
                used[b, h * G + g] = n_used
    return o, used, margin

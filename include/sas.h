/*
 * sas.h - C ABI of the MI355X (gfx950) library for SAS log-gated block-sparse attention.
 *
 * The method (sources are cited by page title and section):
 *   [SAS-ja] "論文解説: SAS — 疎注意の「どのブロックを読むか」を言語モデル損失で端から端まで学習する"
 *            (ta-paperlens.web.app), sections "前提" (paper section 3) and "仕組み"
 *            (paper sections 4.1, 4.3 eq. (9), Algorithm 2 / section 5.1).
 *   [SAS-ko] "SAS는 언어모델 손실로 문맥 순위를 직접 학습하는 사후 어텐션 희소화다"
 *            (onedev.kr/papers/5), sections "어떻게 동작하나" and "무엇과 다른가" (choices 1, 2, 4).
 *
 * A sequence of n tokens is cut into NB = n / 64 blocks. For query block j the history is
 * blocks 0..j-1, scored by s[j][m]. Gates g = softmax(s) over that history; the current
 * block j has gate 1 and a causal mask. The K highest scores pick the history blocks
 * attended; log g of each picked block is added to every logit of its tokens, and the
 * softmax runs over the current block plus the picked blocks. Inference (decode) uses the
 * same Top-K but no gates.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or synchronises. Work is enqueued on `stream` (a hipStream_t passed
 *     as void*, NULL = the null stream) and the call returns without waiting.
 *   - Layouts are row-major and contiguous: Q/O/dO [B][Hq][n][d], K/V [B][Hkv][n][d]
 *     (d innermost), so one 64-token block of one KV head is one contiguous run.
 *     Query head hq uses KV head hq / (Hq / Hkv).
 *   - bf16 tensors are passed as void*; they hold IEEE bfloat16 bit patterns.
 *   - Arguments are checked on the host before anything is enqueued. A failed check
 *     returns a status code with nothing enqueued; sas_last_error() then describes it.
 *     A launch failure returns SAS_ERR_HIP. Faults inside kernels are asynchronous and
 *     surface at the caller's next synchronisation.
 *   - Supported: block == 64, d in {64, 128}, Hq % Hkv == 0, pointers 16-byte aligned.
 *   - Entry points are thread-safe; the library keeps no state between calls except a
 *     thread-local error string.
 */
#ifndef SAS_H
#define SAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SAS_OK = 0,
    SAS_ERR_INVALID_ARG = 1,   /* a pointer, size or value is out of its documented range */
    SAS_ERR_UNSUPPORTED = 2,   /* valid but outside what the kernels implement            */
    SAS_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the size query says   */
    SAS_ERR_HIP = 4            /* a HIP runtime call or launch failed                      */
} sas_status;

typedef enum {
    SAS_SCOPE_SPARSE = 0,      /* keep min(topk, C_j) blocks ([SAS-ko] choice 4, sparse)  */
    SAS_SCOPE_FULL = 1         /* keep every history block ([SAS-ko] choice 4, full)      */
} sas_scope;

typedef enum {
    SAS_ROWS_PREFILL = 0,      /* s[B][H][rows][ld]; row j (query block j) has j valid
                                  history scores in columns 0..j-1                         */
    SAS_ROWS_DECODE = 1        /* s[B][H][rows][ld]; every row of batch entry b has
                                  row_valid[b] valid history scores                       */
} sas_rows;

/* Where the gate enters the attention, [SAS-ko] "무엇과 다른가", choice 1. */
typedef enum {
  SAS_GATE_INSIDE = 0,   /* the method: log g added to the logits inside the softmax */
  SAS_GATE_OUTSIDE = 1   /* the alternative: o = sum_i p_i g_m(i) v_i with p the softmax of
                            the ungated logits (the gate only rescales V) */
} sas_gate_placement;

/* Gate activation phi, [SAS-ko] "무엇과 다른가": choice 2 (the method) and the alternatives
 * the explainer compares it with. */
typedef enum {
  SAS_GATE_SOFTMAX = 0,           /* g = softmax(s) over the row's valid history (choice 2) */
  SAS_GATE_SOFTMAX_SELECTED = 1,  /* softmax over the kept blocks only: the normalisation a
                                     straight-through binary Top-K mask implies (choice 3) */
  SAS_GATE_SIGMOID = 2,           /* g = sigmoid(s) */
  SAS_GATE_EXP = 3                /* the raw score injected as the logit: log g = s */
} sas_gate;

/* Library version string, e.g. "sas-mi355x 0.1.0 gfx950". */
const char* sas_version(void);

/* Human-readable name of a status code. */
const char* sas_status_string(sas_status status);

/* Detail of the last failed call on this thread ("" if none). */
const char* sas_last_error(void);

/*
 * sas_gates - gate normalisation of history scores.
 * [SAS-ko] "무엇과 다른가", choice 2: g = softmax(s), log g_m = s_m - LSE(s) over every valid
 * history block of the row; [SAS-ja] "仕組み": the current block's gate is fixed at 1 and is
 * not part of s.
 *
 *   s          fp32 [B][H][rows][ld], device; only the valid columns of each row are read.
 *   B, H, rows number of batch entries, heads and score rows per head (rows >= 1).
 *   cols       columns per row that may be valid (1 <= cols <= ld, cols <= 8192).
 *              PREFILL requires cols >= rows - 1.
 *   mode       sas_rows; PREFILL: row j has j valid scores. DECODE: row_valid[b] valid
 *              scores for every row of batch entry b (values are clamped to [0, cols]).
 *   row_valid  int32 [B], device; required for DECODE, must be NULL for PREFILL.
 *   lse        fp32 [B][H][rows], device, out: LSE of the valid scores (-inf if none).
 *   g          fp32 [B][H][rows][ld], device, out, nullable: g_m = exp(s_m - LSE) for valid
 *              columns, 0 for columns valid..cols-1; columns >= cols are not written.
 * NaN scores are read as -inf (gate 0).
 */
sas_status sas_gates(const float* s, int B, int H, int rows, int cols, int ld, int mode,
                     const int32_t* row_valid, float* lse, float* g, void* stream);

/*
 * sas_topk_select - softmax gates plus Top-K history-block selection, one row per
 * (batch, head, query block).
 * [SAS-ja] "前提": the selector's K best blocks form the attended set S = B_0 U (U_{m in I} B_m);
 * "仕組み" (Algorithm 2): inference takes the Top-K of s itself; [SAS-ko] choice 2 for the
 * log-gates; choice 4 for the scope.
 *
 * Same s/B/H/rows/cols/ld/mode/row_valid arguments as sas_gates, and:
 *   topk   budget K >= 0 in blocks (ignored for SAS_SCOPE_FULL).
 *   scope  sas_scope. A row keeps k = min(topk, valid) blocks (SPARSE) or valid (FULL).
 *   gate   sas_gate: the activation whose log g is written to logg (selection itself
 *          always ranks the raw scores).
 *   kcap   row stride of idx/logg; must be >= min(topk, V) (SPARSE) or >= V (FULL), where
 *          V = min(cols, rows - 1) in PREFILL mode and V = cols in DECODE mode.
 *   idx    int32 [B][H][rows][kcap], out: the kept block indices in ascending order,
 *          padded with -1. Ties in s go to the lower block index; -0 equals +0; NaN ranks
 *          as -inf. The comparison uses the fp32 scores, so the result is exact.
 *   cnt    int32 [B][H][rows], out: k.
 *   lse    fp32 [B][H][rows], out, nullable: the gate's normaliser: LSE of the row's
 *          valid scores (SOFTMAX), LSE of the kept scores (SOFTMAX_SELECTED; -inf if none),
 *          0 (SIGMOID, EXP).
 *   logg   fp32 [B][H][rows][kcap], out, nullable: log g for each kept block, 0 pad:
 *          s_m - lse (both softmax gates), log sigmoid(s_m), or s_m (EXP); -inf for a NaN
 *          or -inf score.
 */
sas_status sas_topk_select(const float* s, int B, int H, int rows, int cols, int ld, int mode,
                           const int32_t* row_valid, int topk, int scope, int gate, int kcap,
                           int32_t* idx, int32_t* cnt, float* lse, float* logg, void* stream);

/*
 * sas_gates_bwd - gradient with respect to the scores through the gate softmax.
 * [SAS-ko] "무엇과 다른가", choice 2: g = softmax(s) over a row's valid history blocks; the
 * chain rule through its Jacobian diag(g) - g g^T gives, for every valid block m,
 *   ds_m = g_m (dg_m - c),   c = sum over the row's selected slots t of g_idx[t] dg[t],
 * where dg_m is the gradient of block m's gate: dg[t] for the selected block idx[t] and 0
 * for an unselected one (choice 4, sparse scope: only selected blocks reach the attention).
 *
 * Same s/B/H/rows/cols/ld/mode/row_valid arguments as sas_gates, and:
 *   gate   sas_gate used for the forward. SOFTMAX: the formula above. SOFTMAX_SELECTED: the
 *          same Jacobian over the kept blocks only (ds = 0 elsewhere). SIGMOID:
 *          ds_m = dg_m g_m (1 - g_m); EXP: ds_m = dg_m g_m; on kept blocks, 0 elsewhere.
 *   lse    fp32 [B][H][rows], in: the normaliser sas_topk_select wrote for s with the same
 *          gate (NULL allowed for SIGMOID and EXP). For the softmax gates g_m is recomputed
 *          as exp(s_m - lse); a NaN or -inf score, or a row whose lse is -inf, has g = 0
 *          and therefore ds = 0.
 *   idx    int32 [B][H][rows][kcap], in: the selected blocks; entries t < cnt that lie in
 *          [0, valid) must be distinct within a row (sas_topk_select writes them so);
 *          others are ignored.
 *   cnt    int32 [B][H][rows], in: selected slots per row, clamped to [0, kcap].
 *   dg     fp32 [B][H][rows][kcap], in: dL/dg aligned with idx (sas_attn_bwd's dg output,
 *          reshaped; in PREFILL mode H is the KV-head count).
 *   kcap   0..8192; idx and dg may be NULL when kcap = 0.
 *   ds     fp32 [B][H][rows][ld], out: every entry is written (0 for m >= valid). Must
 *          not alias s.
 * Errors: as sas_gates, plus SAS_ERR_INVALID_ARG for a bad gate, a NULL cnt/ds (or lse
 * with a softmax gate), kcap out of range, or ds == s. Deterministic (no atomics to global memory).
 */
sas_status sas_gates_bwd(const float* s, int B, int H, int rows, int cols, int ld, int mode,
                         const int32_t* row_valid, int gate, const float* lse, const int32_t* idx,
                         const int32_t* cnt, const float* dg, int kcap, float* ds, void* stream);

/*
 * sas_attn_fwd - log-gated block-sparse attention forward.
 * [SAS-ja] "仕組み", eq. (9) / [SAS-ko] "어떻게 동작하나": o = softmax(scale q K_S^T + log g_S) V_S
 * with S = the current block (causal, gate 1) plus the blocks in idx, log g broadcast to
 * every token of its block. scale multiplies q.k only; log g is added unscaled.
 *
 *   Q        bf16 [B][Hq][n][d]; K, V bf16 [B][Hkv][n][d].
 *   idx, cnt, logg  as written by sas_topk_select with rows = n / 64, laid out
 *            [B][Hkv][n/64][kcap] and [B][Hkv][n/64]. Rows must hold distinct blocks < j;
 *            entries outside [0, j) are ignored. cnt is clamped to [0, min(kcap, j)].
 *            logg may be NULL: every kept block then has gate 1 (ungated sparse attention).
 *   n        multiple of 64.  d in {64, 128}.  block must be 64.  kcap >= 0.
 *   scale    finite, >= 1e-30 (typically 1/sqrt(d)).
 *   placement sas_gate_placement. OUTSIDE: the softmax runs over the ungated logits of S
 *            (a block whose gate is 0 still counts in the normaliser) and each probability
 *            is multiplied by its block's gate before the V product.
 *   O        bf16 [B][Hq][n][d], out.
 *   lse_rows fp32 [B][Hq][n], out: natural-log softmax normaliser of each query row (of the
 *            ungated logits for OUTSIDE; the backward needs it).
 */
sas_status sas_attn_fwd(const void* Q, const void* K, const void* V, const int32_t* idx,
                        const int32_t* cnt, const float* logg, int B, int Hq, int Hkv, int n,
                        int d, int block, int kcap, float scale, int placement, void* O,
                        float* lse_rows, void* stream);

/* Bytes of device workspace sas_attn_bwd needs for these sizes (0 on invalid sizes). */
size_t sas_attn_bwd_workspace_size(int B, int Hq, int Hkv, int n, int d, int block, int kcap);

/*
 * sas_attn_bwd - backward of sas_attn_fwd, with the gate gradient.
 * Content gradients are those of softmax attention over S (only attended keys receive
 * gradient: [SAS-ko] choice 4, sparse scope). The gate gradient follows [SAS-ko] choice 1:
 * dg_jm = sum over the G*64 query rows t of KV head h's group in block j and keys i of
 * block m of (p~_ti / g_jm) dO_t.(v_i - o_t), i.e. the derivative with respect to g_jm.
 * With placement OUTSIDE the gradients are those of o = sum_i p_i g_m(i) v_i: dV uses the
 * weights p g, dS = p (g dP - delta), and dg_jm = sum_{t, i in B_m} p_ti dO_t.v_i (the
 * gradient the explainer gives for that placement).
 *
 *   Q, K, V, idx, cnt, logg, sizes, scale, placement: exactly as passed to sas_attn_fwd.
 *   O, lse_rows  the forward's outputs. dO bf16 [B][Hq][n][d].
 *   idx rows must be ascending (as sas_topk_select writes them).
 *   dQ fp32 [B][Hq][n][d], dK, dV fp32 [B][Hkv][n][d], out (overwritten, not accumulated).
 *   dg fp32 [B][Hkv][n/64][kcap], out: aligned with idx, 0 on padding slots.
 *   ws, ws_bytes  device workspace of at least sas_attn_bwd_workspace_size() bytes,
 *            16-byte aligned; its contents need no initialisation. It holds the inverse
 *            index, the key-major pass's work plan, the partial dK / dV of key blocks whose
 *            lists are split over several workgroups and per-row delta / LSE values, so
 *            calls that may run at the same time (other streams) need separate workspaces.
 * Returns SAS_ERR_UNSUPPORTED when (Hq / Hkv) * n * d * 2 >= 2^31 (the key-major pass
 * addresses the query rows of one KV group with 31-bit offsets).
 */
sas_status sas_attn_bwd(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* lse_rows, const int32_t* idx,
                        const int32_t* cnt, const float* logg, int B, int Hq, int Hkv, int n,
                        int d, int block, int kcap, float scale, int placement, float* dQ,
                        float* dK, float* dV, float* dg, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace sas_decode needs for these sizes (0 on invalid sizes). */
size_t sas_decode_workspace_size(int B, int Hq, int Hkv, int d, int kcap);

/*
 * sas_decode - one decode step in the inference form ([SAS-ja] "仕組み", Algorithm 2 /
 * section 5.1): ungated sparse attention of each new query token over its current block
 * plus the Top-K blocks chosen by sas_topk_select (mode DECODE, rows = 1,
 * row_valid[b] = (kv_len[b] - 1) / 64).
 *
 *   q        bf16 [B][Hq][d]: the new token's queries.
 *   Kc, Vc   bf16 [B][Hkv][Lmax][d]: the caches, already holding the new token's K/V.
 *            Rows at or past kv_len[b] are never used (they read as zero), so they may
 *            hold anything, NaN included.
 *   kv_len   int32 [B], device: tokens in each cache (1 <= kv_len <= Lmax, clamped). The
 *            query is token kv_len - 1; its current block is tokens
 *            [64 * floor((kv_len - 1) / 64), kv_len).
 *   idx, cnt int32 [B][Hkv][kcap] and [B][Hkv] from sas_topk_select; entries outside
 *            [0, (kv_len - 1) / 64) are ignored.
 *   logg     fp32 [B][Hkv][kcap] or NULL. NULL is the inference form (no gates); a non-NULL
 *            pointer adds the log-gates as in training (useful to check decode against the
 *            training forward).
 *   o        bf16 [B][Hq][d], out.
 *   ws       workspace of sas_decode_workspace_size() bytes, 16-byte aligned; it holds the
 *            partial softmax states of split block lists (no initialisation needed), so
 *            calls that may run at the same time need separate workspaces.
 * Returns SAS_ERR_UNSUPPORTED when Hq / Hkv > 32 or Lmax * d * 2 >= 2^31.
 */
sas_status sas_decode(const void* q, const void* Kc, const void* Vc, const int32_t* kv_len,
                      int Lmax, const int32_t* idx, const int32_t* cnt, const float* logg,
                      int B, int Hq, int Hkv, int d, int block, int kcap, float scale, void* o,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * sas_decode_topk - one decode step with its block selection in the same launch
 * ([SAS-ja] "仕組み", Algorithm 2: Top-K of the history scores, then ungated attention
 * over the current block and the kept blocks). Per (sequence, KV head) the kept blocks are
 * exactly those sas_topk_select picks in mode DECODE (rows = 1, row_valid[b] =
 * (kv_len[b] - 1) / 64, K = topk: ties to the lower index, -0 equal to +0, NaN ranked as
 * -inf), and o is bit-identical to sas_topk_select followed by sas_decode. The selection
 * overlaps the copies of the current block and saves the selection launch.
 *
 *   s        fp32 [B][Hkv][ld]: history block scores; row (b, h) reads its first
 *            (kv_len[b] - 1) / 64 entries.
 *   ld       row pitch of s, >= (Lmax - 1) / 64.
 *   topk     K, 1 <= K <= 64.
 *   idx, cnt int32 [B][Hkv][topk] and [B][Hkv], out, nullable (both or neither): the kept
 *            blocks as sas_topk_select writes them (ascending, -1 padded) and their number.
 *   q, Kc, Vc, kv_len, Lmax, B, Hq, Hkv, d, block, scale, o: as for sas_decode.
 *   ws       workspace of sas_decode_workspace_size(B, Hq, Hkv, d, topk) bytes.
 * Returns SAS_ERR_UNSUPPORTED for topk > 64 or (Lmax - 1) / 64 > 1024 (rows of more than
 * 1024 history blocks); sas_topk_select and sas_decode cover those.
 */
sas_status sas_decode_topk(const void* q, const void* Kc, const void* Vc, const int32_t* kv_len,
                           int Lmax, const float* s, int ld, int topk, int B, int Hq, int Hkv,
                           int d, int block, float scale, void* o, int32_t* idx, int32_t* cnt,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * sas_decode_noalloc - sas_decode for callers that cannot allocate device memory: code
 * being captured into a HIP graph, tight serving loops, harnesses that forbid allocation.
 * Same computation, arguments, results and launches as sas_decode, without the workspace
 * arguments: the partial softmax states of split block lists go to a 16 MiB scratch array
 * that the library holds on each device it runs on (until the process ends). The call
 * itself allocates nothing (no hipMalloc, hipFree or allocating library routine); its
 * first call on a device looks up that device's scratch address (hipGetSymbolAddress) and
 * keeps it.
 * The scratch needs B * Hkv * chunks * (Hq / Hkv) * (d + 2) * 4 bytes, where the launch
 * splits each (sequence, KV head) list into chunks only when B * Hkv < 512 (then about
 * 512 workgroups in all): at most ~17 MB for Hq / Hkv = 32, d = 128. Sizes whose launch
 * would need more than the 16 MiB are rejected with SAS_ERR_UNSUPPORTED and nothing is
 * enqueued. The scratch needs no initialisation (every chunk writes its whole partial).
 * Every call on one device shares that device's scratch: calls that may overlap on one
 * device (other streams, other threads) race and must be serialised by the caller.
 */
sas_status sas_decode_noalloc(const void* q, const void* Kc, const void* Vc, const int32_t* kv_len,
                              int Lmax, const int32_t* idx, const int32_t* cnt, const float* logg,
                              int B, int Hq, int Hkv, int d, int block, int kcap, float scale, void* o,
                              void* stream);

/*
 * sas_decode_early_stop - sas_decode with a mass-threshold early stop over the selected
 * blocks, the rule of [S2O-ja] "S2O: オンライン置換によるスパースアテンションの早期停止"
 * (section "2. 早期停止ルール"; prior art, used as a budget rule on top of Top-K).
 * Per query head: the current block first, then the kept blocks in descending order key
 * (ties to the lower block index); each block is attended, and the head takes no further
 * block once the block's softmax mass is below tau times the mass accumulated before it.
 * tau = 0 gives sas_decode (ungated) over every kept block.
 *
 *   q, Kc, Vc, kv_len, Lmax, idx, cnt, sizes, block, scale, o: as sas_decode.
 *   kcap     at most 63 (the list of a (sequence, KV head) is sorted inside one wave).
 *   order    fp32 [B][Hkv][kcap], device: the score (or log-gate) of each kept block; only
 *            its order matters. NaN orders as -inf.
 *   tau      finite, >= 0.
 *   used     int32 [B][Hq], device, out, nullable: history blocks each head attended.
 * No workspace: one workgroup walks each (sequence, KV head) list.
 */
sas_status sas_decode_early_stop(const void* q, const void* Kc, const void* Vc, const int32_t* kv_len,
                                 int Lmax, const int32_t* idx, const int32_t* cnt, const float* order,
                                 int B, int Hq, int Hkv, int d, int block, int kcap, float scale,
                                 float tau, void* o, int32_t* used, void* stream);

/*
 * sas_decode_paged - sas_decode over a paged KV cache (serving layout).
 * Same computation as sas_decode ([SAS-ja] "仕組み", Algorithm 2); the cache is a pool of
 * pages of 64 tokens (one SAS block each) and a page table per sequence:
 *   Kpool, Vpool  bf16 [num_pages][Hkv][64][d], device, 16-byte aligned.
 *   page_table    int32 [B][max_pages], device: page of logical block m of sequence b,
 *                 read for m <= (kv_len[b] - 1) / 64 (the current block and every block
 *                 idx may name). A page id outside [0, num_pages) makes that block read
 *                 as empty (weight 0).
 *   kv_len        int32 [B], device, clamped to [1, 64 * max_pages].
 * Rows of the current page at or past kv_len are never read (they read as zero), so a
 * page allocator may leave them unwritten. Other arguments and the workspace as
 * sas_decode (kcap, idx, cnt, logg, scale, o, ws).
 */
sas_status sas_decode_paged(const void* q, const void* Kpool, const void* Vpool, int num_pages,
                            const int32_t* page_table, int max_pages, const int32_t* kv_len,
                            const int32_t* idx, const int32_t* cnt, const float* logg, int B, int Hq,
                            int Hkv, int d, int block, int kcap, float scale, void* o, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * sas_decode_paged_topk - sas_decode_topk over a paged KV cache: one decode step with its
 * block selection in the same launch ([SAS-ja] "仕組み", Algorithm 2), the caches laid out
 * as for sas_decode_paged. The kept blocks are those sas_topk_select picks in mode DECODE
 * (rows = 1, row_valid[b] = (kv_len[b] - 1) / 64, K = topk), and o is bit-identical to
 * sas_topk_select followed by sas_decode_paged.
 *
 *   s        fp32 [B][Hkv][ld]: history block scores (logical block order); row (b, h)
 *            reads its first (kv_len[b] - 1) / 64 entries.
 *   ld       row pitch of s, >= max_pages - 1.
 *   topk     K, 1 <= K <= 64.
 *   idx, cnt int32 [B][Hkv][topk] and [B][Hkv], out, nullable (both or neither): the kept
 *            logical blocks (ascending, -1 padded) and their number.
 *   Kpool, Vpool, num_pages, page_table, max_pages, kv_len: as for sas_decode_paged.
 *   q, B, Hq, Hkv, d, block, scale, o: as for sas_decode.
 *   ws       workspace of sas_decode_workspace_size(B, Hq, Hkv, d, topk) bytes.
 * Returns SAS_ERR_UNSUPPORTED for topk > 64 or max_pages > 1025 (rows of more than 1024
 * history blocks); sas_topk_select and sas_decode_paged cover those.
 */
sas_status sas_decode_paged_topk(const void* q, const void* Kpool, const void* Vpool, int num_pages,
                                 const int32_t* page_table, int max_pages, const int32_t* kv_len,
                                 const float* s, int ld, int topk, int B, int Hq, int Hkv, int d,
                                 int block, float scale, void* o, int32_t* idx, int32_t* cnt, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * sas_pool_keys - block means of a decode key cache, the input of sas_decode_select.
 * kbar_m = (1/64) sum of the 64 keys of block m, summed in fp32 and rounded to bf16
 * (nearest even). In serving, call it with first_block = the first block completed since
 * the last call; a block is pooled once, when it is complete.
 *
 *   Kc          bf16 [B][Hkv][Lmax][d], device, 16-byte aligned.
 *   Lmax        multiple of 64; C = Lmax / 64 blocks per (sequence, KV head).
 *   d           64 or 128.
 *   kv_len      int32 [B], device: tokens in each sequence's cache.
 *   first_block blocks m in [first_block, C) with (m + 1) * 64 <= kv_len[b] are pooled.
 *   kbar        bf16 [B][Hkv][C][d], device, 16-byte aligned, out; other blocks untouched.
 */
sas_status sas_pool_keys(const void* Kc, int B, int Hkv, int Lmax, int d, const int32_t* kv_len,
                         int first_block, void* kbar, void* stream);

/*
 * sas_decode_select - block scores and Top-K blocks for one decode step (long contexts).
 * The pages leave the selector network undefined; the block score stands in for it as the
 * mean attention score over the block ([PBS-ja] "Sparser Block-Sparse Attention via Token
 * Permutation", sections 3 and 4: block importance by mean pooling), averaged over the G
 * query heads of the KV group:
 *   s[b][h][m] = scale * qbar . kbar_m,  qbar = (1/G) sum_g q[b][hG+g],
 * for the history blocks m < V_b = (kv_len[b] - 1) / 64 (clamped to [0, C]). Selection then
 * follows [SAS-ja] "仕組み" Algorithm 2 exactly as sas_topk_select in DECODE / SPARSE mode:
 * the k = min(topk, V_b) largest s (ties to the lower index, -0 equals +0, NaN as -inf),
 * ascending, -1 pad; the comparison uses the fp32 scores written to s.
 *
 *   q       bf16 [B][Hq][d], device.   kbar  bf16 [B][Hkv][C][d] from sas_pool_keys.
 *   C       blocks per row of kbar and s, 1..8192.   d  64 or 128.   Hq % Hkv == 0.
 *   kv_len  int32 [B], device.   scale  finite, > 0 (1/sqrt(d) for the attention scale).
 *   topk    >= 0.   kcap  row stride of idx / logg, in [min(topk, C), 8192].
 *   s       fp32 [B][Hkv][C], device, out: entries m < V_b written, the rest untouched.
 *   idx     int32 [B][Hkv][kcap], out.   cnt  int32 [B][Hkv], out: k.
 *   lse     fp32 [B][Hkv], out, nullable: LSE of the row's V_b scores (-inf if none).
 *   logg    fp32 [B][Hkv][kcap], out, nullable: s - LSE per kept block, 0 pad.
 * Two kernels on the stream: block scores (rows x chunks of the pooled cache), then one
 * workgroup per row for the Top-K. No workspace beyond s.
 */
sas_status sas_decode_select(const void* q, const void* kbar, int B, int Hq, int Hkv, int d, int C,
                             const int32_t* kv_len, float scale, int topk, int kcap, float* s,
                             int32_t* idx, int32_t* cnt, float* lse, float* logg, void* stream);

/* Bytes of device workspace sas_decode_long needs (0 on invalid or unsupported sizes). */
size_t sas_decode_long_workspace_size(int B, int Hq, int Hkv, int d, int C, int topk);

/*
 * sas_decode_long - one decode step over a long context in two launches: the block scores
 * of sas_decode_select with their Top-K, and the decode of sas_decode ([SAS-ja] "仕組み",
 * Algorithm 2; the scores as in sas_decode_select, [PBS-ja] sections 3 and 4). The kept
 * blocks and o are identical to sas_decode_select (kcap = topk) followed by sas_decode.
 * The first launch scores the pooled keys in chunks and keeps each chunk's min(topk,
 * blocks) best (every block of the row's Top-K is among its chunk's best); the decode
 * ranks those candidates in its own prologue, beside the copies of the current block,
 * instead of a row-wide selection launch.
 *
 *   q, Kc, Vc, kv_len, Lmax, B, Hq, Hkv, d, block, scale, o: as for sas_decode.
 *   kbar     bf16 [B][Hkv][C][d] from sas_pool_keys, 16-byte aligned; C in [(Lmax - 1) / 64,
 *            8192].
 *   topk     K, 1 <= K <= 64.
 *   idx, cnt int32 [B][Hkv][topk] and [B][Hkv], out, nullable (both or neither): the kept
 *            blocks (ascending, -1 padded) and their number, as sas_decode_select writes them.
 *   ws       workspace of sas_decode_long_workspace_size(B, Hq, Hkv, d, C, topk) bytes,
 *            16-byte aligned (partial states and candidates; no initialisation needed).
 * Returns SAS_ERR_UNSUPPORTED for topk > 64 or C > 8192.
 */
sas_status sas_decode_long(const void* q, const void* kbar, int C, const void* Kc, const void* Vc,
                           const int32_t* kv_len, int Lmax, int topk, int B, int Hq, int Hkv, int d,
                           int block, float scale, void* o, int32_t* idx, int32_t* cnt, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * sas_pool_keys_paged - sas_pool_keys over a paged key cache (the layout of
 * sas_decode_paged): kbar[b][h][m] is the mean of the 64 keys of page page_table[b][m],
 * summed in the same order (so equal, bit for bit, to sas_pool_keys on the same keys laid
 * out contiguously). A page id outside [0, num_pages) pools to zero.
 *
 *   Kpool       bf16 [num_pages][Hkv][64][d], device, 16-byte aligned.
 *   page_table  int32 [B][max_pages], device.   max_pages <= 8192; C = max_pages.
 *   kv_len, first_block, d: as for sas_pool_keys.
 *   kbar        bf16 [B][Hkv][max_pages][d], device, 16-byte aligned, out; other blocks untouched.
 */
sas_status sas_pool_keys_paged(const void* Kpool, int num_pages, const int32_t* page_table, int max_pages,
                               int B, int Hkv, int d, const int32_t* kv_len, int first_block, void* kbar,
                               void* stream);

/*
 * sas_decode_long_paged - sas_decode_long over a paged KV cache: the same candidates
 * launch on kbar (from sas_pool_keys_paged, C = max_pages), then the paged decode ranking
 * them. Kept blocks and o are identical to sas_decode_select (kcap = topk) followed by
 * sas_decode_paged.
 *
 *   Kpool, Vpool, num_pages, page_table, max_pages, kv_len: as for sas_decode_paged
 *   (max_pages <= 8192).
 *   kbar     bf16 [B][Hkv][max_pages][d], 16-byte aligned.
 *   q, topk, B, Hq, Hkv, d, block, scale, o, idx, cnt: as for sas_decode_long.
 *   ws       workspace of sas_decode_long_workspace_size(B, Hq, Hkv, d, max_pages, topk) bytes.
 */
sas_status sas_decode_long_paged(const void* q, const void* kbar, const void* Kpool, const void* Vpool,
                                 int num_pages, const int32_t* page_table, int max_pages,
                                 const int32_t* kv_len, int topk, int B, int Hq, int Hkv, int d, int block,
                                 float scale, void* o, int32_t* idx, int32_t* cnt, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * Kernel timing, for measurement (not part of the pages' method; off by default).
 *
 * sas_profile_enable(on): while on, every kernel the library launches is bracketed by two
 * HIP events recorded on the stream it is launched on (the library creates and keeps the
 * events; enabling itself makes no HIP call). Returns SAS_OK.
 *
 * sas_profile_collect: waits for the events recorded since the last collect, sums the
 * elapsed time per kernel and writes up to `max` entries in first-launch order:
 *   names     max * name_len chars, out (NUL-terminated names; may be NULL),
 *   launches  int[max], out (may be NULL): launches of each kernel,
 *   total_ms  double[max], out (may be NULL): summed event time of each kernel.
 * Returns the number of entries written, or -1 if an event query failed. The record is
 * cleared either way. Kernel names: select, fwd, inv_count, inv_scan (the inverse-index
 * offsets and the key-major pass's work plan), inv_fill, dq, dg_reduce, dkv, dkv_reduce,
 * gates_bwd, decode, decode_merge, pool, block_scores, topk_rows.
 */
sas_status sas_profile_enable(int on);
int sas_profile_collect(int max, char* names, int name_len, int* launches, double* total_ms);

/*
 * sas_profile_only(name): while timing is on, bracket only the kernels of this name (one of
 * the names listed above; NULL or "" brackets every kernel again). Each bracketed launch
 * adds two event records to its stream; timing one kernel of a multi-kernel step keeps the
 * others free of them. The name is copied (at most 31 characters). Returns SAS_OK, or
 * SAS_ERR_INVALID_ARG for a longer name.
 */
sas_status sas_profile_only(const char* name);

/*
 * sas_profile_collect_launches: like sas_profile_collect, but one entry per recorded launch
 * in launch order (names as above, ms[i] its event time), for medians and percentiles. At
 * most `max` entries are written; the record is cleared either way. Returns the count, or
 * -1 if an event query failed.
 */
int sas_profile_collect_launches(int max, char* names, int name_len, double* ms);

/*
 * sas_debug_workgroup_order - a debugging aid (not part of the pages' method): with seed != 0,
 * the attention forward, both backward passes and decode take their work items in a
 * permuted order (work item = (workgroup * mul + add) mod grid, mul coprime with the grid
 * size, both derived from the seed); seed 0 (the default) restores the natural order.
 * Results do not depend on the order (every output element has one producer and a fixed
 * reduction order), which the determinism tests check with it. Library-wide setting,
 * read at each launch; returns SAS_OK.
 */
sas_status sas_debug_workgroup_order(unsigned long long seed);

/*
 * Measurement microkernels (not part of the pages' method): what the chip delivers, so
 * achieved rates can be quoted against measured peaks beside the vendor's.
 *
 * sas_measure_mfma: `workgroups` workgroups of 4 waves, each wave running `iters` rounds of
 * 8 independent bf16 32x32x16 MFMAs (32768 FLOP each), i.e. workgroups * 4 * iters * 8 *
 * 32768 FLOP in all; the caller times the launch with events on `stream`. clocks: device
 * uint64 [2 * workgroups], out: per workgroup, the shader-clock cycles (s_memtime) and the
 * constant 100 MHz counter ticks (s_memrealtime) of wave 0's loop, so clock = cycles /
 * ticks * 100 MHz. sink: device float[1], never written in practice.
 *
 * sas_measure_read: one streaming read of `bytes` (a multiple of 16; buf 16-byte aligned)
 * with 16-byte loads from 4096 workgroups; sink as above.
 *
 * Both return SAS_ERR_INVALID_ARG on a NULL pointer or a non-positive size, SAS_ERR_HIP on
 * a launch failure.
 */
sas_status sas_measure_mfma(int workgroups, int iters, unsigned long long* clocks, float* sink, void* stream);
sas_status sas_measure_read(const void* buf, size_t bytes, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAS_H */

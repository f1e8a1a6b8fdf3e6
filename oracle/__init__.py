"""CPU oracle for SAS log-gated block-sparse attention (test infrastructure only; see
``sas_oracle``)."""
from .sas_oracle import (GATES, NEG_INF, attn_bwd, attn_fwd, bwd_query_block, decode,  # noqa: F401
                         decode_block_scores, decode_early_stop, decode_paged, decode_rows_valid, decode_select, fwd_query_block,
                         gates_bwd, gates_bwd_prefill, gather_pages, dense_causal, pool_keys, row_log_gates,
                         row_log_gates_variant, row_topk, select, select_prefill)

"""CPU oracle for SAS log-gated block-sparse attention (test infrastructure only; see
``sas_oracle``)."""
from .sas_oracle import (NEG_INF, attn_bwd, attn_fwd, decode, decode_rows_valid,  # noqa: F401
                         dense_causal, row_log_gates, row_topk, select, select_prefill)

"""CPU oracle for the CSA lightning-indexer top-k step (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It shares no code with the HIP library.
"""
from .csa_oracle import (  # noqa: F401
    decode_bf16, widen, visible_count, row_scores, order_desc, select_topk,
    oracle_topk, oracle_threshold, oracle_interleaved, oracle_recall,
    logit_threshold, exact_int_scores, exhaustive_topk,
    row_score_vector, RowScorer,
)
from .csa_attention_oracle import attention_row, oracle_attention  # noqa: F401
from .csa_union_oracle import oracle_union, oracle_multilayer  # noqa: F401
from .csa_projection_oracle import (  # noqa: F401
    project, project_abs, oracle_query, oracle_head_weights, oracle_compress_keys,
)

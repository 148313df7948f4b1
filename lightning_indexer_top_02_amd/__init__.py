"""MI355X (gfx950) CSA lightning-indexer top-k.

    I[t, s] = sum_j w[t, j] * max(q[t, j] . k[s], 0),  top-k keys per query row.

The compute runs in libcsa_indexer.so (HIP kernels behind a C ABI, declared
in include/csa_indexer.h); this package only marshals torch tensors into it.
"""
from ._binding import (  # noqa: F401
    CSA_BF16, CSA_F32, CSA_NONCAUSAL, CSA_SORTED, EXPORTS, LIB_PATH, MAX_DECODE_SQ, MAX_TOPK,
    NOALLOC_SCRATCH_BYTES, OP_DECODE, OP_INTERLEAVED, OP_PREFILL, OP_RECALL, OP_THRESHOLD, CsaError, CsaProblem,
    index_threshold_select, index_topk_decode, index_topk_decode_noalloc, index_topk_interleaved, index_topk_prefill,
    load_library, make_problem, set_recall, version, workspace_size,
    CsaAttnProblem, attention_workspace_size, make_attn_problem, sparse_attention, union_rows,
    MultiLayerSelector, MAX_LAYERS, batchable_layers, index_threshold_select_layers, MultiLayerIndexer,
    project, query_projection, head_weight_projection, compress_keys, test_options,
)

"""fp64 CPU oracle (test infrastructure only; never on the product path)."""
from .elastic_oracle import (  # noqa: F401
    allowed, as_f64, attention, attention_kv, block_list_from_pattern, block_list_resolve,
    block_streaming, chunked_prefill, decode_bf16,
    effective_flops, effective_sparsity, entries, head_modes, lse_merge, mean_exact, mean_f64,
    model_sparsity_ratio, pooled_rows, retrieval_scores, route, row_key_counts,
    static_assignment,
)

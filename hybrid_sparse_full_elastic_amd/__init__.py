"""Elastic Attention prefill on MI355X (gfx950): Python binding of libelastic.

Argument marshalling only: every step of the path (router pooling and MLP, scheduling,
hybrid-head attention) runs in the HIP kernels of ``libelastic.so`` behind the C ABI in
``include/elastic.h``.  torch supplies device memory and streams.  There is no fallback:
if the library is missing, importing this package raises.
"""
from ._binding import (  # noqa: F401
    ABI_VERSION, ElasticError, LIB_PATH, SparseCfg, attn_entries, attn_prefill, attn_prefill_kv,
    attn_workspace_size, block_list_entries, lib, lse_merge, retrieval_scores,
    retrieval_workspace_size, route, route_workspace_size, sparse_cfg, static_assignment,
)

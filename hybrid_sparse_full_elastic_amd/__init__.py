"""Elastic Attention prefill on MI355X (gfx950): Python binding of libelastic.

Argument marshalling only: every step of the path (router pooling and MLP, scheduling,
hybrid-head attention) runs in the HIP kernels of ``libelastic.so`` behind the C ABI in
``include/elastic.h``.  torch supplies device memory and streams.  There is no fallback: the
library is loaded on first use (``lib`` or any call), and that raises if it is missing, so
``python -m hybrid_sparse_full_elastic_amd.build`` works on a clean checkout.
"""
from ._binding import (  # noqa: F401
    ABI_VERSION, ElasticError, LIB_PATH, SparseCfg, attn_entries, attn_prefill, attn_prefill_kv,
    attn_prefill_noalloc,
    attn_workspace_size, block_list_entries, lse_merge, retrieval_scores,
    retrieval_workspace_size, route, route_workspace_size, sparse_cfg, static_assignment,
)


def __getattr__(name):
    if name == "lib":  # the loaded C library
        from ._binding import _lib
        return _lib()
    raise AttributeError(name)

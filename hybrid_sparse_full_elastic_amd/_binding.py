"""ctypes binding of libelastic (see include/elastic.h for the contract of each call).

Argument marshalling only: shapes, dtypes and devices are checked here, then every call goes
to the C ABI.  The library is loaded on first use; if it is missing the call raises."""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libelastic.so")
ABI_VERSION = 4

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
BF16, FP32 = 0, 1
STREAMING, BLOCK, BLOCK_LIST = 0, 1, 2


class ElasticError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        L = _lib()
        msg = f"{where}: {L.elastic_status_string(status).decode()}"
        if status == EHIP or (status == EWORKSPACE and "noalloc" in where):
            msg += f" ({L.elastic_last_error().decode()})"
        super().__init__(msg)


class SparseCfg(C.Structure):
    _fields_ = [("kind", C.c_int32), ("sink_tokens", C.c_int32), ("window_tokens", C.c_int32),
                ("block_size", C.c_int32), ("sink_blocks", C.c_int32),
                ("local_blocks", C.c_int32), ("stride_blocks", C.c_int32),
                ("list_qblocks", C.c_int32), ("list_row_ptr", C.c_void_p),
                ("list_col_idx", C.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m hybrid_sparse_full_elastic_amd.build`")
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
    L.elastic_abi_version.restype = C.c_int
    L.elastic_abi_version.argtypes = []
    L.elastic_status_string.restype = C.c_char_p
    L.elastic_status_string.argtypes = [C.c_int]
    L.elastic_last_error.restype = C.c_char_p
    L.elastic_last_error.argtypes = []
    L.elastic_route_workspace_size.restype = sz
    L.elastic_route_workspace_size.argtypes = [i32, i64, i32]
    L.elastic_route.restype = C.c_int
    L.elastic_route.argtypes = [vp, i32, vp, i32, i64, i32, i32, i32, vp, i32, vp, i32, f32, vp, vp,
                                vp, sz, vp]
    L.elastic_attn_workspace_size.restype = sz
    L.elastic_attn_workspace_size.argtypes = [i32, i32, i64, i32, i32, i32]
    L.elastic_attn_prefill.restype = C.c_int
    L.elastic_attn_prefill.argtypes = [vp, vp, vp, vp, i32, vp, i32, i64, i32, i32, i32, i32, f32,
                                       vp, C.POINTER(SparseCfg), vp, vp, sz, vp]
    L.elastic_attn_prefill_noalloc.restype = C.c_int
    L.elastic_attn_prefill_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, i32, i64, i32, i32, i32, i32,
                                               f32, vp, C.POINTER(SparseCfg), vp, vp]
    L.elastic_attn_prefill_kv.restype = C.c_int
    L.elastic_attn_prefill_kv.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, i64, i64, i32, i32, i32,
                                          i32, i32, i32, i32, f32, vp, C.POINTER(SparseCfg), vp, vp,
                                          sz, vp]
    L.elastic_lse_merge.restype = C.c_int
    L.elastic_lse_merge.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, vp]
    L.elastic_attn_entries.restype = C.c_int
    L.elastic_attn_entries.argtypes = [C.POINTER(i32), i32, C.POINTER(i32), i32, i32,
                                       C.POINTER(SparseCfg), C.POINTER(i64)]
    L.elastic_attn_entries_lists.restype = C.c_int
    L.elastic_attn_entries_lists.argtypes = [C.POINTER(i32), i32, C.POINTER(i32), i32, i32, i32,
                                             i32, C.POINTER(i32), C.POINTER(i32), C.POINTER(i64)]
    L.elastic_retrieval_workspace_size.restype = sz
    L.elastic_retrieval_workspace_size.argtypes = [i32, i32, i32]
    L.elastic_retrieval_scores.restype = C.c_int
    L.elastic_retrieval_scores.argtypes = [vp, vp, i32, vp, i32, i64, i32, i32, i32, i32, f32, vp,
                                           vp, vp, vp, sz, vp]
    L.elastic_static_assignment.restype = C.c_int
    L.elastic_static_assignment.argtypes = [vp, i32, C.c_double, vp, vp]
    if L.elastic_abi_version() != ABI_VERSION:
        raise ImportError(f"libelastic ABI {L.elastic_abi_version()} != binding ABI {ABI_VERSION}")
    return L


_LIB = None


def _lib():
    """The loaded library (loaded on first use)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def sparse_cfg(d: Optional[dict]) -> Optional[SparseCfg]:
    """SparseCfg from a pattern dict: {"kind": "streaming", "sink", "window"} or
    {"kind": "block", "block", "sink_blocks", "local_blocks", "stride_blocks"}."""
    if d is None:
        return None
    if isinstance(d, SparseCfg):
        return d
    if d["kind"] == "streaming":
        return SparseCfg(STREAMING, int(d["sink"]), int(d["window"]), 0, 0, 0, 0)
    if d["kind"] == "block":
        return SparseCfg(BLOCK, 0, 0, int(d["block"]), int(d["sink_blocks"]),
                         int(d["local_blocks"]), int(d["stride_blocks"]))
    if d["kind"] == "block_list":
        # CSR of key-block indices on the device; the struct keeps the tensors alive
        rp, ci = d["row_ptr"], d["col_idx"]
        for name, t in (("row_ptr", rp), ("col_idx", ci)):
            if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.int32 and t.is_contiguous()):
                raise ValueError(f"block_list {name} must be a contiguous int32 device tensor")
        cfg = SparseCfg(BLOCK_LIST, 0, 0, int(d["block"]), 0, 0, 0, int(d["qblocks"]),
                        rp.data_ptr(), ci.data_ptr() if ci.numel() > 0 else rp.data_ptr())
        cfg._keep = (rp, ci)
        return cfg
    raise ValueError(f"unknown sparse kind {d['kind']!r}")


def _i32_array(values):
    vals = [int(x) for x in values]
    return (C.c_int32 * max(1, len(vals)))(*vals)


def block_list_entries(seqlens, head_mask, n_q_heads: int, n_kv_heads: int, lists: dict) -> int:
    """Allowed score entries for a block-list pattern, counted by the library from a host copy
    of the CSR lists.  Full heads count n(n+1)/2 each."""
    def host(x):
        return x.cpu().tolist() if isinstance(x, torch.Tensor) else [int(v) for v in x]
    rp, ci = host(lists["row_ptr"]), host(lists["col_idx"])
    rows = len(seqlens) * n_kv_heads * int(lists["qblocks"])
    if len(rp) != rows + 1 or (len(rp) > 0 and len(ci) < rp[-1]):
        raise ValueError(f"block lists need row_ptr of {rows + 1} entries and col_idx of row_ptr[-1]")
    mask_arr = None
    if head_mask is not None:
        mask_arr = _i32_array(int(x) for row in head_mask for x in row)
    out = C.c_int64(0)
    st = _lib().elastic_attn_entries_lists(_i32_array(seqlens), len(seqlens), mask_arr, n_q_heads,
                                           n_kv_heads, int(lists["block"]), int(lists["qblocks"]),
                                           _i32_array(rp), _i32_array(ci), C.byref(out))
    if st != OK:
        raise ElasticError(st, "elastic_attn_entries_lists")
    return int(out.value)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _check_dev(name, t, dtype=None, shape=None, device=None):
    """Device, contiguity, dtype and (when given) exact shape and device of a tensor argument:
    the kernels read and write whole [rows, ...] extents, so a smaller tensor would be
    overrun on the device."""
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _seq_args(cu_seqlens: Optional[torch.Tensor], total: int, device=None):
    if cu_seqlens is None:
        return 1
    _check_dev("cu_seqlens", cu_seqlens, torch.int32, device=device)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be int32 [batch + 1] with batch >= 1")
    return cu_seqlens.numel() - 1


def _workspace(workspace, need: int, device):
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _check_dev("workspace", workspace, device=device)
    return workspace


def _check_qkv(q, k, v, what="T"):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, device=q.device)
        if t.dim() != 3:
            raise ValueError(f"{name} must be [{what}, heads, head_dim]")
    if q.dtype not in (torch.bfloat16, torch.float32) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype bf16 or fp32")


def _check_lists(sparse, batch: int, n_kv_heads: int, device):
    """Block lists on the device: the row pointers must cover every (sequence, KV head, query
    block) row the kernels may read."""
    if isinstance(sparse, dict) and sparse.get("kind") == "block_list":
        rp = sparse["row_ptr"]
        rows = batch * n_kv_heads * int(sparse["qblocks"])
        _check_dev("block_list row_ptr", rp, torch.int32, (rows + 1,), device)
        _check_dev("block_list col_idx", sparse["col_idx"], torch.int32, device=device)


def route_workspace_size(batch: int, total_tokens: int, d_model: int) -> int:
    return int(_lib().elastic_route_workspace_size(batch, total_tokens, d_model))


def route(hidden: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor,
          cu_seqlens: Optional[torch.Tensor] = None, threshold: float = 0.0,
          pool_head: int = 0, pool_tail: int = 0, logits: Optional[torch.Tensor] = None,
          mask: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
          stream=None):
    """Attention Router on device: returns (logits [B, Hkv] fp32, mask [B, Hkv] int32)."""
    _check_dev("hidden", hidden)
    _check_dev("w1", w1, torch.float32)
    _check_dev("w2", w2, torch.float32)
    if hidden.dtype not in (torch.bfloat16, torch.float32) or hidden.dim() != 2:
        raise ValueError("hidden must be a 2-D bf16 or fp32 tensor [T, d_model]")
    T, d = hidden.shape
    dev = hidden.device
    B = _seq_args(cu_seqlens, T, dev)
    if w1.dim() != 2 or w2.dim() != 2:
        raise ValueError("w1 must be [d_router, d_model] and w2 [n_kv_heads, d_router]")
    dr, hkv = w1.shape[0], w2.shape[0]
    _check_dev("w1", w1, torch.float32, (dr, d), dev)
    _check_dev("w2", w2, torch.float32, (hkv, dr), dev)
    if logits is None:
        logits = torch.empty((B, hkv), dtype=torch.float32, device=dev)
    if mask is None:
        mask = torch.empty((B, hkv), dtype=torch.int32, device=dev)
    _check_dev("logits", logits, torch.float32, (B, hkv), dev)
    _check_dev("mask", mask, torch.int32, (B, hkv), dev)
    workspace = _workspace(workspace, route_workspace_size(B, T, d), dev)
    st = _lib().elastic_route(_ptr(hidden), BF16 if hidden.dtype == torch.bfloat16 else FP32,
                           _ptr(cu_seqlens), B, T, d, pool_head, pool_tail, _ptr(w1), dr,
                           _ptr(w2), hkv, float(threshold), _ptr(logits), _ptr(mask),
                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                           _stream(stream))
    if st != OK:
        raise ElasticError(st, "elastic_route")
    return logits, mask


def attn_workspace_size(dtype: int, batch: int, total_tokens: int, n_q_heads: int,
                        n_kv_heads: int, head_dim: int) -> int:
    return int(_lib().elastic_attn_workspace_size(dtype, batch, total_tokens, n_q_heads, n_kv_heads,
                                               head_dim))


def attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
                 head_mask: Optional[torch.Tensor] = None, sparse=None,
                 softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 stream=None):
    """Hybrid-head GQA prefill: returns o [T, Hq, D] (and fills ``lse`` [Hq, T] if given)."""
    _check_qkv(q, k, v)
    T, hq, D = q.shape
    hkv = k.shape[1]
    if k.shape != (T, hkv, D) or v.shape != (T, hkv, D):
        raise ValueError("k and v must be [T, n_kv_heads, head_dim] matching q")
    dev = q.device
    B = _seq_args(cu_seqlens, T, dev)
    dtype = BF16 if q.dtype == torch.bfloat16 else FP32
    if out is None:
        out = torch.empty_like(q)
    _check_dev("out", out, q.dtype, q.shape, dev)
    _check_dev("lse", lse, torch.float32, (hq, T), dev)
    _check_dev("head_mask", head_mask, torch.int32, (B, hkv), dev)
    _check_lists(sparse, B, hkv, dev)
    workspace = _workspace(workspace, attn_workspace_size(dtype, B, T, hq, hkv, D), dev)
    cfg = sparse_cfg(sparse)
    st = _lib().elastic_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), dtype, _ptr(cu_seqlens), B,
                                  T, int(max_seqlen if max_seqlen is not None else T), hq, hkv, D,
                                  float(softmax_scale), _ptr(head_mask),
                                  C.byref(cfg) if cfg is not None else None, _ptr(lse),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    if st != OK:
        raise ElasticError(st, "elastic_attn_prefill")
    return out


def attn_prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                         cu_seqlens: Optional[torch.Tensor] = None,
                         max_seqlen: Optional[int] = None, head_mask: Optional[torch.Tensor] = None,
                         sparse=None, softmax_scale: float = 0.0,
                         lse: Optional[torch.Tensor] = None, stream=None):
    """attn_prefill for callers that cannot allocate: no workspace (the library's per-GPU
    scheduler scratch is used) and the caller provides ``out``.  Calls that overlap on one GPU
    race on that scratch."""
    _check_qkv(q, k, v)
    T, hq, D = q.shape
    hkv = k.shape[1]
    if k.shape != (T, hkv, D) or v.shape != (T, hkv, D):
        raise ValueError("k and v must be [T, n_kv_heads, head_dim] matching q")
    dev = q.device
    B = _seq_args(cu_seqlens, T, dev)
    _check_dev("out", out, q.dtype, q.shape, dev)
    _check_dev("lse", lse, torch.float32, (hq, T), dev)
    _check_dev("head_mask", head_mask, torch.int32, (B, hkv), dev)
    _check_lists(sparse, B, hkv, dev)
    cfg = sparse_cfg(sparse)
    st = _lib().elastic_attn_prefill_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), BF16 if q.dtype == torch.bfloat16 else FP32,
        _ptr(cu_seqlens), B, T, int(max_seqlen if max_seqlen is not None else T), hq, hkv, D,
        float(softmax_scale), _ptr(head_mask), C.byref(cfg) if cfg is not None else None,
        _ptr(lse), _stream(stream))
    if st != OK:
        raise ElasticError(st, "elastic_attn_prefill_noalloc")
    return out


def attn_prefill_kv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    cu_seqlens_q: Optional[torch.Tensor] = None,
                    cu_seqlens_k: Optional[torch.Tensor] = None,
                    max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
                    q_pos: int = -1, k_pos: int = 0, head_mask: Optional[torch.Tensor] = None,
                    sparse=None, softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None):
    """Query rows against a separate range of key rows (chunked prefill, key-range splits):
    returns o [Tq, Hq, D].  q_pos -1 = queries are the last key positions of each sequence."""
    _check_qkv(q, k, v, "rows")
    Tq, hq, D = q.shape
    Tk, hkv = k.shape[0], k.shape[1]
    if k.shape != (Tk, hkv, D) or v.shape != (Tk, hkv, D):
        raise ValueError("k and v must be [Tk, n_kv_heads, head_dim] with q's head_dim")
    dev = q.device
    B = _seq_args(cu_seqlens_q, Tq, dev)
    if (cu_seqlens_k is None) != (cu_seqlens_q is None) or (cu_seqlens_k is not None and _seq_args(cu_seqlens_k, Tk, dev) != B):
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be given, for the same batch")
    dtype = BF16 if q.dtype == torch.bfloat16 else FP32
    if out is None:
        out = torch.empty_like(q)
    _check_dev("out", out, q.dtype, q.shape, dev)
    _check_dev("lse", lse, torch.float32, (hq, Tq), dev)
    _check_dev("head_mask", head_mask, torch.int32, (B, hkv), dev)
    _check_lists(sparse, B, hkv, dev)
    workspace = _workspace(workspace, attn_workspace_size(dtype, B, Tq, hq, hkv, D), dev)
    cfg = sparse_cfg(sparse)
    st = _lib().elastic_attn_prefill_kv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), dtype, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Tq,
        Tk, int(max_seqlen_q if max_seqlen_q is not None else Tq),
        int(max_seqlen_k if max_seqlen_k is not None else Tk), int(q_pos), int(k_pos), hq, hkv, D,
        float(softmax_scale), _ptr(head_mask), C.byref(cfg) if cfg is not None else None, _ptr(lse),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if st != OK:
        raise ElasticError(st, "elastic_attn_prefill_kv")
    return out


def lse_merge(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor,
              out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
              stream=None):
    """Merge two attention results over disjoint key sets; in place when out is o_a."""
    dev = o_a.device
    _check_dev("o_a", o_a)
    if o_a.dim() != 3 or o_a.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("o_a must be a bf16 or fp32 [rows, heads, head_dim] tensor")
    rows, heads, D = o_a.shape
    _check_dev("o_b", o_b, o_a.dtype, o_a.shape, dev)
    _check_dev("lse_a", lse_a, torch.float32, (heads, rows), dev)
    _check_dev("lse_b", lse_b, torch.float32, (heads, rows), dev)
    if out is None:
        out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    _check_dev("out", out, o_a.dtype, o_a.shape, dev)
    _check_dev("lse_out", lse_out, torch.float32, (heads, rows), dev)
    dtype = BF16 if o_a.dtype == torch.bfloat16 else FP32
    st = _lib().elastic_lse_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(out),
                               _ptr(lse_out), dtype, rows, heads, D, _stream(stream))
    if st != OK:
        raise ElasticError(st, "elastic_lse_merge")
    return out, lse_out


def retrieval_workspace_size(batch: int, max_seqlen: int, n_q_heads: int) -> int:
    return int(_lib().elastic_retrieval_workspace_size(batch, max_seqlen, n_q_heads))


def retrieval_scores(q: torch.Tensor, k: torch.Tensor, needle: torch.Tensor,
                     cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
                     softmax_scale: float = 0.0, workspace: Optional[torch.Tensor] = None,
                     stream=None):
    """Attention mass of each sequence's last token on its needle span: returns
    (scores_q [B, Hq], scores_kv [B, Hkv]) fp32.  ``needle`` is int32 [B, 2] (begin, end)."""
    for name, t in (("q", q), ("k", k)):
        _check_dev(name, t, device=q.device)
        if t.dim() != 3:
            raise ValueError(f"{name} must be [T, heads, head_dim]")
    if q.dtype not in (torch.bfloat16, torch.float32) or k.dtype != q.dtype:
        raise ValueError("q and k must share dtype bf16 or fp32")
    T, hq, D = q.shape
    hkv = k.shape[1]
    if k.shape != (T, hkv, D):
        raise ValueError("k must be [T, n_kv_heads, head_dim] matching q")
    B = _seq_args(cu_seqlens, T, q.device)
    _check_dev("needle", needle, torch.int32, (B, 2), q.device)
    ms = int(max_seqlen if max_seqlen is not None else T)
    sq = torch.empty((B, hq), dtype=torch.float32, device=q.device)
    skv = torch.empty((B, hkv), dtype=torch.float32, device=q.device)
    workspace = _workspace(workspace, retrieval_workspace_size(B, ms, hq), q.device)
    dtype = BF16 if q.dtype == torch.bfloat16 else FP32
    st = _lib().elastic_retrieval_scores(_ptr(q), _ptr(k), dtype, _ptr(cu_seqlens), B, T, ms, hq, hkv,
                                      D, float(softmax_scale), _ptr(needle), _ptr(sq), _ptr(skv),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream))
    if st != OK:
        raise ElasticError(st, "elastic_retrieval_scores")
    return sq, skv


def static_assignment(scores: torch.Tensor, omega_msr: float, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Full (1) / sparse (0) mask of the same shape as ``scores`` (fp32, any shape, e.g.
    [layers, n_kv_heads]): the floor((1 - omega_msr) * N) highest scores stay full."""
    _check_dev("scores", scores, torch.float32)
    if out is None:
        out = torch.empty(scores.shape, dtype=torch.int32, device=scores.device)
    _check_dev("out", out, torch.int32, scores.shape, scores.device)
    st = _lib().elastic_static_assignment(_ptr(scores), scores.numel(), float(omega_msr), _ptr(out),
                                       _stream(stream))
    if st != OK:
        raise ElasticError(st, "elastic_static_assignment")
    return out


def attn_entries(seqlens, head_mask, n_q_heads: int, n_kv_heads: int, sparse=None) -> int:
    """Allowed score entries over all query heads (host closed forms, no GPU involved)."""
    if isinstance(sparse, dict) and sparse.get("kind") == "block_list":
        return block_list_entries(seqlens, head_mask, n_q_heads, n_kv_heads, sparse)
    lens = (C.c_int32 * len(seqlens))(*[int(x) for x in seqlens])
    mask_arr = None
    if head_mask is not None:
        flat = [int(x) for row in head_mask for x in row]
        mask_arr = (C.c_int32 * len(flat))(*flat)
    cfg = sparse_cfg(sparse)
    out = C.c_int64(0)
    st = _lib().elastic_attn_entries(lens, len(seqlens), mask_arr, n_q_heads, n_kv_heads,
                                  C.byref(cfg) if cfg is not None else None, C.byref(out))
    if st != OK:
        raise ElasticError(st, "elastic_attn_entries")
    return int(out.value)

"""fp64 CPU oracle for Elastic Attention's prefill path (router + hybrid-head GQA attention).

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain definition that the GPU
library is checked against.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import or call it; the product path never
does, and it shares no code with the HIP library.

Source: "Elastic Attention: Test-time Adaptive Sparsity Ratios for Efficient
Transformers" (arXiv 2601.17367), as summarised on paperlayer.ai
(abs/2601.17367v2).  Sections cited below are that summary's headings.

What is computed (readings of points the summary leaves open are marked READING):

* Router (section 1 "Introduction": head-wise routing from the layer's input hidden
  states; section 3 "Attention Router": pooled states -> task/router MLP -> head-wise
  logits -> binary full/sparse choice per KV head).
  READING: the pooled state is the arithmetic mean of the layer-input hidden
  states over all tokens of a sequence (boundary pooling of the first/last tokens,
  appendix H.4 "Router Input Length", is selectable with ``pool_head/pool_tail``);
  the MLP is z = W1 h, a = ReLU(z), l = W2 a with no biases; a KV head is FULL
  iff l > threshold (ties go to sparse).  Column sums are fp64 (``exact=True``:
  correctly rounded with ``math.fsum``).
* Allowed key sets (section 2 "Hybrid Head Mechanism"; section 4 and appendix B.2
  for streaming sparse attention; appendix D.1 "Sparse Inference" for block
  sparsity).  Positions are local to a sequence; every set contains j = i.
    full:       {j <= i}
    streaming:  {j <= i : j < sink  or  i - j < window}            (READING: window includes i)
    block:      {j <= i : j//B in K(i//B)},  K(qb) = {kb < sink_blocks}
                  U {qb-local_blocks .. qb}  U {kb : stride > 0 and kb % stride == 0}
  Query head h reads KV head h // G (GQA, repeat_kv convention) and takes that KV
  head's mode (section 3 "Attention Router": one decision per key-value head).
* Attention: exact two-pass softmax over the allowed set, s_j = scale <q_i, k_j>,
  scale = D^-1/2 unless given; o_i = sum_j softmax(s)_j v_j; lse_i = m + log sum exp(s - m).
  Head outputs are concatenated (o is [T, Hq, D]).
* Counters: entries (allowed (query, key) pairs over all query heads), effective
  FLOPs = 4*D*entries, model sparsity ratio (fraction of sparse heads) and effective
  sparsity (section 2 "Sparsity Ratio Computation").
* Deployment forms (appendix D.1 "Sparse Inference": block-sparse streaming with block
  64 and 128 sink tokens, prefill in chunks of 16,384 queries):
    attention_kv     queries at absolute positions attend a range of keys at absolute
                     positions; the allowed sets above are evaluated on absolute positions
                     and restricted to the keys present.  A row that sees no key has
                     o = 0 and lse = -inf.
    lse_merge        the plain identity for softmax attention over two disjoint key sets:
                     lse = log(e^a + e^b),  o = e^(a - lse) o_a + e^(b - lse) o_b.
    chunked_prefill  each query chunk attends every key up to its own end (the queries
                     are the last positions of the keys), chunk results concatenated.
    block lists      READING (explicit per-head block lists, the consumer half of
                     content-based block selection): the key blocks query block qb of KV head
                     g in sequence b may see are given explicitly, key blocks after qb are
                     ignored (causal), and a query sees key j iff j <= i and j's block is
                     listed for i's block.  An empty list leaves the row without keys.
    block_streaming  READING: the block-granular form of sink + window streaming is the
                     block pattern with block 64, ceil(sink / 64) sink blocks, a window of
                     window / 64 blocks that includes the query's own block, and no stride.
* Static retrieval-score head assignment (appendix C.1 "Retrieval Score Calculation"):
    retrieval_scores   S = attention mass of a sequence's last token on the needle positions,
                       sum over j in needle of softmax_j(scale <q_last, k_j>) over all keys
                       of the sequence (the last token sees every key).  READING: the needle
                       is one contiguous span [begin, end) of key positions (clipped to the
                       sequence); a KV head's score is the mean of its G query heads' scores;
                       an empty sequence scores 0.
    static_assignment  k = floor((1 - omega_msr) * N) of the N (layer, KV head) units with
                       the highest scores stay full, the rest sparse.  READING: k in fp64;
                       equal scores rank by lower unit index; NaN ranks below every number.
"""
from __future__ import annotations

import math
from contextlib import nullcontext
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

try:  # keep BLAS single-threaded inside the oracle's own thread pool
    from threadpoolctl import threadpool_limits
except Exception:  # pragma: no cover
    threadpool_limits = None


# ----------------------------------------------------------------------------- inputs
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bfloat16 bit patterns (uint16)."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray) -> np.ndarray:
    """uint16 arrays are bf16 bit patterns; float arrays are taken at face value."""
    if x.dtype == np.uint16:
        return decode_bf16(x)
    return np.asarray(x, dtype=np.float64)


def _seq_bounds(cu_seqlens: Optional[Sequence[int]], total: int) -> np.ndarray:
    if cu_seqlens is None:
        return np.array([0, total], dtype=np.int64)
    return np.asarray(cu_seqlens, dtype=np.int64)


# ----------------------------------------------------------------------------- router
def pooled_rows(n: int, pool_head: int = 0, pool_tail: int = 0) -> np.ndarray:
    """Local row indices the router pools for a sequence of length n.

    0,0 -> every row.  Otherwise the first ``pool_head`` and the last ``pool_tail``
    rows (appendix H.4, boundary pooling); when they overlap, each row counts once."""
    if pool_head == 0 and pool_tail == 0:
        return np.arange(n)
    rows = set(range(min(n, pool_head))) | set(range(max(0, n - pool_tail), n))
    return np.array(sorted(rows), dtype=np.int64)


def mean_exact(x: np.ndarray) -> np.ndarray:
    """Column means of a 2-D float array with correctly rounded column sums (math.fsum)."""
    n, d = x.shape
    out = np.empty(d, dtype=np.float64)
    step = 256
    for c0 in range(0, d, step):
        cols = np.ascontiguousarray(x[:, c0:c0 + step].T).tolist()
        for c, col in enumerate(cols):
            out[c0 + c] = math.fsum(col) / n
    return out


def mean_f64(x: np.ndarray, rows: np.ndarray, chunk: int = 8192) -> np.ndarray:
    """Column means of rows ``rows`` of ``x`` (bf16 bits or floats): fp64 sums, row by row.

    The rounding error of the sum is at most len(rows) * 2**-53 * sum|x| per column, about
    1e-9 of the pooled value at 131K rows: far below the 1e-3 logit band the router
    comparison exempts.  ``route(..., exact=True)`` uses ``mean_exact`` instead."""
    total = np.zeros(x.shape[1], dtype=np.float64)
    for r0 in range(0, len(rows), chunk):
        total += as_f64(x[rows[r0:r0 + chunk]]).sum(axis=0)
    return total / max(len(rows), 1)


def route(hidden: np.ndarray, cu_seqlens, w1: np.ndarray, w2: np.ndarray,
          threshold: float = 0.0, pool_head: int = 0, pool_tail: int = 0,
          exact: bool = False) -> dict:
    """Attention Router forward for every sequence of a packed batch.

    hidden [T, d] (bf16 bits or float), w1 [d_router, d], w2 [Hkv, d_router].
    Returns pooled [B, d], hidden-layer z [B, d_router], logits [B, Hkv] (fp64) and
    mask [B, Hkv] int32 with 1 = full attention, 0 = sparse attention."""
    x = hidden
    W1 = np.asarray(w1, dtype=np.float64)
    W2 = np.asarray(w2, dtype=np.float64)
    cu = _seq_bounds(cu_seqlens, x.shape[0])
    B = len(cu) - 1
    pooled = np.zeros((B, x.shape[1]))
    z = np.zeros((B, W1.shape[0]))
    logits = np.zeros((B, W2.shape[0]))
    for b in range(B):
        n = int(cu[b + 1] - cu[b])
        rows = pooled_rows(n, pool_head, pool_tail) + cu[b]
        if len(rows) == 0:
            pooled[b] = 0.0                      # nothing to pool: logits 0, all sparse
        elif exact:
            pooled[b] = mean_exact(as_f64(x[rows]))
        else:
            pooled[b] = mean_f64(x, rows)
        z[b] = W1 @ pooled[b]
        a = np.maximum(z[b], 0.0)
        logits[b] = W2 @ a
    mask = (logits > threshold).astype(np.int32)
    return {"pooled": pooled, "z": z, "logits": logits, "mask": mask}


# ----------------------------------------------------------------------------- masks
def allowed(i, j, full: bool, sparse: Optional[dict]) -> np.ndarray:
    """Boolean (broadcast over i, j): may query position i attend key position j?"""
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    causal = j <= i
    if full:
        return causal
    kind = sparse["kind"]
    if kind == "streaming":
        return causal & ((j < sparse["sink"]) | (i - j < sparse["window"]))
    if kind == "block":
        B = sparse["block"]
        qb, kb = i // B, j // B
        keep = (kb < sparse["sink_blocks"]) | (qb - kb <= sparse["local_blocks"])
        stride = sparse["stride_blocks"]
        if stride > 0:
            keep = keep | (kb % stride == 0)
        return causal & keep
    if kind == "block_set":  # one (sequence, KV head) of a block-list pattern, resolved
        B = sparse["block"]
        vis = sparse["visible"]  # bool [query blocks, key blocks]
        qb, kb = i // B, j // B
        inside = (qb < vis.shape[0]) & (kb < vis.shape[1]) & (qb >= 0) & (kb >= 0)
        got = np.zeros(np.broadcast(qb, kb).shape, dtype=bool)
        qq, kk = np.broadcast_arrays(qb, kb)
        got[inside] = vis[qq[inside], kk[inside]]
        return causal & got
    raise ValueError(f"unknown sparse kind {kind!r}")


def block_list_resolve(sparse: dict, b: int, g: int, n_kv_heads: int) -> dict:
    """The block set of sequence b, KV head g from a block-list pattern:
    {"kind": "block_list", "block": B, "row_ptr": [B*Hkv*nqb + 1], "col_idx": [...], "qblocks": nqb}
    (CSR rows r = (b * Hkv + g) * nqb + qb, key block indices per row)."""
    nqb = int(sparse["qblocks"])
    rp = np.asarray(sparse["row_ptr"], dtype=np.int64)
    ci = np.asarray(sparse["col_idx"], dtype=np.int64)
    vis = np.zeros((nqb, nqb), dtype=bool)
    for qb in range(nqb):
        r = (b * n_kv_heads + g) * nqb + qb
        kb = ci[rp[r]:rp[r + 1]]
        kb = kb[(kb >= 0) & (kb <= qb)]   # later blocks are ignored (causal)
        vis[qb, kb] = True
    return {"kind": "block_set", "block": int(sparse["block"]), "visible": vis}


def block_list_from_pattern(pattern: dict, batch: int, n_kv_heads: int, n_max: int) -> dict:
    """The block lists that reproduce a fixed block pattern (every sequence and head alike)."""
    B = pattern["block"]
    nqb = -(-n_max // B)
    rows = []
    for qb in range(nqb):
        i = qb * B + B - 1
        kb = np.arange(qb + 1)
        keep = allowed(np.full(qb + 1, i), kb * B, False, pattern)
        rows.append(kb[keep])
    row_ptr, col = [0], []
    for _ in range(batch * n_kv_heads):
        for r in rows:
            col.extend(int(x) for x in r)
            row_ptr.append(len(col))
    return {"kind": "block_list", "block": B, "qblocks": nqb, "row_ptr": row_ptr, "col_idx": col}


def row_key_counts(n: int, full: bool, sparse: Optional[dict], rows=None,
                   block_rows: int = 256) -> np.ndarray:
    """|A(i)| for the given local rows (default all), by enumerating the mask."""
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty(len(rows), dtype=np.int64)
    for r0 in range(0, len(rows), block_rows):
        ii = rows[r0:r0 + block_rows]
        jj = np.arange(int(ii.max()) + 1)
        out[r0:r0 + block_rows] = allowed(ii[:, None], jj[None, :], full, sparse).sum(axis=1)
    return out


def head_modes(head_mask, batch: int, n_kv_heads: int) -> np.ndarray:
    """[B, Hkv] bool, True = full.  ``None`` means every head is full."""
    if head_mask is None:
        return np.ones((batch, n_kv_heads), dtype=bool)
    return np.asarray(head_mask).reshape(batch, n_kv_heads) != 0


def entries(seqlens, head_mask, sparse, n_q_heads: int, n_kv_heads: int) -> int:
    """Allowed (query, key) pairs summed over all query heads and sequences."""
    G = n_q_heads // n_kv_heads
    modes = head_modes(head_mask, len(seqlens), n_kv_heads)
    lists = sparse is not None and sparse.get("kind") == "block_list"
    cache = {}
    total = 0
    for b, n in enumerate(seqlens):
        for g in range(n_kv_heads):
            if lists and not modes[b, g]:
                sp = block_list_resolve(sparse, b, g, n_kv_heads)
                total += G * int(row_key_counts(int(n), False, sp).sum())
                continue
            key = (int(n), bool(modes[b, g]))
            if key not in cache:
                cache[key] = int(row_key_counts(int(n), key[1], sparse).sum())
            total += G * cache[key]
    return total


def effective_flops(n_entries: int, head_dim: int) -> int:
    """Q.K^T and P.V each cost 2*D FLOPs per allowed score entry."""
    return 4 * head_dim * n_entries


def model_sparsity_ratio(head_mask, seqlens=None, token_weighted: bool = False) -> float:
    """Fraction of sparse heads (optionally weighting each sequence by its length)."""
    m = np.asarray(head_mask) != 0
    if not token_weighted:
        return float((~m).sum() / m.size)
    w = np.asarray(seqlens, dtype=np.float64)[:, None]
    return float(((~m) * w).sum() / (w.sum() * m.shape[1]))


def effective_sparsity(seqlens, head_mask, sparse, n_q_heads, n_kv_heads) -> float:
    """1 - (allowed entries) / (entries of all-full causal attention)."""
    dense = sum(n_q_heads * n * (n + 1) // 2 for n in seqlens)
    return 1.0 - entries(seqlens, head_mask, sparse, n_q_heads, n_kv_heads) / dense


# ----------------------------------------------------------------------------- attention
def _attend_block(Q, K, V, ii, full, sparse, scale):
    """Rows ``ii`` (local positions) of one query head: exact two-pass softmax.  A row with
    no allowed key (possible only with explicit block lists) gets o = 0, lse = -inf."""
    jj = np.arange(int(ii.max()) + 1)
    A = allowed(ii[:, None], jj[None, :], full, sparse)
    cols = np.nonzero(A.any(axis=0))[0]
    o = np.zeros((len(ii), V.shape[1]))
    lse = np.full(len(ii), -np.inf)
    if len(cols) == 0:
        return o, lse
    A = A[:, cols]
    s = scale * (Q[ii] @ K[cols].T)
    s = np.where(A, s, -np.inf)
    has = A.any(axis=1)
    m = np.where(has, s.max(axis=1), 0.0)[:, None]
    p = np.exp(s - m)                      # exp(-inf) = 0 for disallowed keys
    denom = p.sum(axis=1, keepdims=True)
    o[has] = (p[has] @ V[cols]) / denom[has]
    lse[has] = m[has, 0] + np.log(denom[has, 0])
    return o, lse


def attention(q, k, v, cu_seqlens, head_mask, sparse, scale: Optional[float] = None,
              rows=None, heads=None, block_rows: int = 64, workers: int = 1):
    """Hybrid-head GQA prefill attention.

    q [T, Hq, D], k/v [T, Hkv, D] (bf16 bit patterns or floats); head_mask [B, Hkv]
    (1 = full; None = all full); sparse = pattern dict for the sparse heads.
    ``rows``: sorted global token indices to evaluate (default all); ``heads``:
    query heads to evaluate (default all).  Returns o [len(rows), len(heads), D]
    and lse [len(heads), len(rows)] in float64."""
    Qa, Ka, Va = as_f64(q), as_f64(k), as_f64(v)
    T, Hq, D = Qa.shape
    Hkv = Ka.shape[1]
    G = Hq // Hkv
    scale = D ** -0.5 if scale is None or scale <= 0 else float(scale)
    cu = _seq_bounds(cu_seqlens, T)
    B = len(cu) - 1
    modes = head_modes(head_mask, B, Hkv)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    seq_of = np.searchsorted(cu, rows, side="right") - 1
    o = np.zeros((len(rows), len(heads), Va.shape[2]))
    lse = np.zeros((len(heads), len(rows)))

    tasks = []
    for b in range(B):
        sel = np.nonzero(seq_of == b)[0]
        if len(sel) == 0:
            continue
        for hi, h in enumerate(heads):
            for r0 in range(0, len(sel), block_rows):
                tasks.append((b, hi, h, sel[r0:r0 + block_rows]))

    def run(task):
        b, hi, h, sel = task
        lo, hi_tok = int(cu[b]), int(cu[b + 1])
        g = h // G
        Q = Qa[lo:hi_tok, h, :]
        K = Ka[lo:hi_tok, g, :]
        V = Va[lo:hi_tok, g, :]
        sp = block_list_resolve(sparse, b, g, Hkv) if sparse is not None and sparse.get("kind") == "block_list" else sparse
        ob, lb = _attend_block(Q, K, V, rows[sel] - lo, bool(modes[b, g]), sp, scale)
        o[sel, hi, :] = ob
        lse[hi, sel] = lb

    if workers <= 1:
        for t in tasks:
            run(t)
    else:
        limit = threadpool_limits(limits=1) if threadpool_limits is not None else nullcontext()
        with limit, ThreadPoolExecutor(workers) as ex:
            list(ex.map(run, tasks))
    return o, lse


# ----------------------------------------------------------------------------- deployment forms
def block_streaming(sink_tokens: int = 128, window_tokens: int = 1024, block: int = 64) -> dict:
    """Block-granular streaming pattern (appendix D.1: block 64, 128 sink tokens)."""
    if window_tokens % block or window_tokens < block:
        raise ValueError("window must be a positive multiple of the block size")
    return {"kind": "block", "block": block, "sink_blocks": -(-sink_tokens // block),
            "local_blocks": window_tokens // block - 1, "stride_blocks": 0}


def _attend_block_abs(Q, K, V, pi, pj, full, sparse, scale):
    """Query rows at absolute positions ``pi`` over keys at absolute positions ``pj``."""
    A = allowed(pi[:, None], pj[None, :], full, sparse)
    cols = np.nonzero(A.any(axis=0))[0]
    o = np.zeros((len(pi), V.shape[1]))
    lse = np.full(len(pi), -np.inf)
    if len(cols) == 0:
        return o, lse
    A = A[:, cols]
    s = scale * (Q @ K[cols].T)
    s = np.where(A, s, -np.inf)
    has = A.any(axis=1)
    m = np.where(has, s.max(axis=1), 0.0)[:, None]
    p = np.exp(s - m)                      # exp(-inf) = 0 for disallowed keys
    denom = p.sum(axis=1, keepdims=True)
    o[has] = (p[has] @ V[cols]) / denom[has]
    lse[has] = m[has, 0] + np.log(denom[has, 0])
    return o, lse


def attention_kv(q, k, v, cu_q, cu_k, head_mask, sparse, scale: Optional[float] = None,
                 q_pos=None, k_pos: int = 0, heads=None, block_rows: int = 64):
    """Queries of sequence b (rows cu_q[b]..cu_q[b+1]) sit at absolute positions
    q_pos[b] + t; its keys (rows cu_k[b]..cu_k[b+1] of k/v) at k_pos + j.  ``q_pos`` None
    means the queries are the last positions of the keys (q_pos[b] = k_pos + n_k - n_q).
    Returns o [Tq, len(heads), D] and lse [len(heads), Tq] (natural log)."""
    Qa, Ka, Va = as_f64(q), as_f64(k), as_f64(v)
    Tq, Hq, D = Qa.shape
    Hkv = Ka.shape[1]
    G = Hq // Hkv
    scale = D ** -0.5 if scale is None or scale <= 0 else float(scale)
    cq = _seq_bounds(cu_q, Tq)
    ck = _seq_bounds(cu_k, Ka.shape[0])
    B = len(cq) - 1
    modes = head_modes(head_mask, B, Hkv)
    heads = list(range(Hq)) if heads is None else list(heads)
    o = np.zeros((Tq, len(heads), Va.shape[2]))
    lse = np.full((len(heads), Tq), -np.inf)
    for b in range(B):
        nq, nk = int(cq[b + 1] - cq[b]), int(ck[b + 1] - ck[b])
        if nq == 0:
            continue
        qp = (k_pos + nk - nq) if q_pos is None else int(np.asarray(q_pos).reshape(-1)[b])
        pj = k_pos + np.arange(nk)
        for hi, h in enumerate(heads):
            g = h // G
            K = Ka[ck[b]:ck[b + 1], g, :]
            V = Va[ck[b]:ck[b + 1], g, :]
            for r0 in range(0, nq, block_rows):
                t = np.arange(r0, min(nq, r0 + block_rows))
                sp = (block_list_resolve(sparse, b, g, Hkv)
                      if sparse is not None and sparse.get("kind") == "block_list" else sparse)
                ob, lb = _attend_block_abs(Qa[cq[b] + t, h, :], K, V, qp + t, pj,
                                           bool(modes[b, g]), sp, scale)
                o[cq[b] + t, hi, :] = ob
                lse[hi, cq[b] + t] = lb
    return o, lse


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Combine attention over two disjoint key sets: o [rows, heads, D], lse [heads, rows]."""
    a = np.asarray(lse_a, dtype=np.float64)
    b = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(a, b)                # -inf when both are -inf
    fin = np.isfinite(lse)
    safe = np.where(fin, lse, 0.0)
    wa = np.where(fin, np.exp(np.where(fin, a, 0.0) - safe), 0.0)
    wb = np.where(fin, np.exp(np.where(fin, b, 0.0) - safe), 0.0)
    o = wa.T[:, :, None] * as_f64(o_a) + wb.T[:, :, None] * as_f64(o_b)
    return o, lse


def chunked_prefill(q, k, v, cu_seqlens, head_mask, sparse, chunk: int,
                    scale: Optional[float] = None, heads=None):
    """Prefill in query chunks: chunk c of sequence b attends its keys up to the chunk's end."""
    Qa = as_f64(q)
    T = Qa.shape[0]
    cu = _seq_bounds(cu_seqlens, T)
    Hq = Qa.shape[1] if heads is None else len(heads)
    o = np.zeros((T, Hq, as_f64(v).shape[2]))
    lse = np.full((Hq, T), -np.inf)
    mask = None if head_mask is None else np.asarray(head_mask).reshape(len(cu) - 1, -1)
    for b in range(len(cu) - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        for c0 in range(lo, hi, chunk):
            c1 = min(hi, c0 + chunk)
            ob, lb = attention_kv(q[c0:c1], k[lo:c1], v[lo:c1], None, None,
                                  None if mask is None else mask[b:b + 1], sparse, scale,
                                  heads=heads)
            o[c0:c1] = ob
            lse[:, c0:c1] = lb
    return o, lse



# ----------------------------------------------------------------------------- static assignment
def retrieval_scores(q, k, cu_seqlens, needle, scale: Optional[float] = None):
    """Appendix C.1 "Retrieval Score Calculation": for each sequence b and query head h, the
    softmax weight that the last token of b puts on the needle span needle[b] = (begin, end)
    (local key positions, clipped to the sequence), over all keys of b.

    Returns (scores_q [B, Hq], scores_kv [B, Hkv]); a KV head's score is the mean over its
    query heads.  Two-pass softmax in fp64: m = max_j s_j, S = sum_needle e^(s_j - m) /
    sum_all e^(s_j - m)."""
    Q, K = as_f64(q), as_f64(k)
    T, Hq, D = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    sc = D ** -0.5 if scale is None else scale
    cu = _seq_bounds(cu_seqlens, T)
    B = len(cu) - 1
    nd = np.asarray(needle, dtype=np.int64).reshape(B, 2)
    sq = np.zeros((B, Hq))
    for b in range(B):
        lo, hi = int(cu[b]), int(cu[b + 1])
        n = hi - lo
        if n == 0:
            continue
        a, e = max(0, int(nd[b, 0])), min(n, int(nd[b, 1]))
        for h in range(Hq):
            s = sc * (K[lo:hi, h // G, :] @ Q[hi - 1, h, :])
            w = np.exp(s - s.max())
            sq[b, h] = (w[a:e].sum() if e > a else 0.0) / w.sum()
    skv = sq.reshape(B, Hkv, G).mean(axis=2)
    return sq, skv


def static_assignment(scores, omega_msr: float) -> np.ndarray:
    """Appendix C.1 "Sparsity Assignment": of the N units (all layers' KV heads, flattened in
    order) the k = floor((1 - omega_msr) * N) with the highest scores stay full (mask 1), the
    rest are sparse (0).  Ties rank by lower index; NaN ranks below every number."""
    s = np.asarray(scores, dtype=np.float64).reshape(-1)
    n = s.size
    k = int(math.floor((1.0 - float(omega_msr)) * n))
    k = max(0, min(n, k))
    key = np.where(np.isnan(s), -np.inf, s)
    nan = np.isnan(s)
    # descending score; NaN after -inf; then ascending index
    order = sorted(range(n), key=lambda i: (nan[i], -key[i], i))
    mask = np.zeros(n, dtype=np.int32)
    mask[order[:k]] = 1
    return mask.reshape(np.shape(scores))

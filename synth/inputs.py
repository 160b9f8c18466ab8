"""Seeded synthetic workloads for hybrid-head GQA prefill (Elastic Attention).

This module draws numbers, rounds them to the storage dtype and packs them.
It holds none of the method's arithmetic (no pooling, routing, masking or
softmax): the fp64 CPU oracle and the GPU library both receive exactly the
arrays built here, so input quantisation is never counted as kernel error.

Random stream definition (both sides depend only on the produced arrays):
a tensor is filled in row-major order in blocks of ``BLOCK = 2**22`` elements;
block ``c`` is ``numpy.random.default_rng([seed, tag, c]).standard_normal(n,
dtype=float32)``, multiplied by ``scale`` in fp32 and, for bf16 tensors,
rounded to bfloat16 with round-to-nearest-even.  Tags: q=0, k=1, v=2,
hidden=3, w1=4, w2=5.

Workloads mirror the shapes the Elastic Attention paper targets (GQA
backbones such as Llama-3.1-8B and Qwen3, long-context prefill from 8K to
131K tokens, streaming sink+window and block-sparse sparse heads; paperlayer
summary of arXiv 2601.17367, sections 2-4 and appendix D.1).  The paper's
benchmark suites (LongBench-E, RULER, LongBench-v2) are not available; these
synthetic tensors stand in for their length mix only.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK = 1 << 22
TAG_Q, TAG_K, TAG_V, TAG_HIDDEN, TAG_W1, TAG_W2 = 0, 1, 2, 3, 4, 5


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw_f32(seed: int, tag: int, shape, scale: float = 1.0) -> np.ndarray:
    """fp32 N(0,1)*scale draws of ``shape`` from the blocked stream above."""
    shape = (int(shape),) if np.isscalar(shape) else tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)
    nblk = (n + BLOCK - 1) // BLOCK
    sc = np.float32(scale)

    def fill(c: int) -> None:
        lo, hi = c * BLOCK, min(n, (c + 1) * BLOCK)
        rng = np.random.default_rng([int(seed), int(tag), c])
        seg = out[lo:hi]
        rng.standard_normal(hi - lo, dtype=np.float32, out=seg)
        if sc != np.float32(1.0):
            np.multiply(seg, sc, out=seg)

    if nblk <= 1:
        for c in range(nblk):
            fill(c)
    else:
        with ThreadPoolExecutor(min(_workers(), nblk)) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of fp32 ``x``, round-to-nearest-even.

    Inputs here are finite normal draws, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 24
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    for lo in range(0, flat_u.size, step):
        seg = flat_u[lo:lo + step]
        lsb = (seg >> np.uint32(16)) & np.uint32(1)
        flat_o[lo:lo + step] = ((seg + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return out


def draw_bf16_bits(seed: int, tag: int, shape, scale: float = 1.0) -> np.ndarray:
    return round_bf16_bits(draw_f32(seed, tag, shape, scale))


@dataclass(frozen=True)
class Workload:
    """One layer's prefill problem. Token-major layouts: q/o [T,Hq,D], k/v [T,Hkv,D]."""
    name: str
    dtype: str                      # "bf16" or "f32"
    seqlens: tuple
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    qkv_scale: float
    qkv_seed: int
    sparse: dict                    # {"kind": "streaming", sink, window} or {"kind": "block", ...}
    router: Optional[dict] = None   # d_model, d_router, w_std, w_seed, hidden_seeds, threshold
    forced_mask: Optional[tuple] = None  # per-sequence tuple of per-KV-head ints, 1 = full
    note: str = ""

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def batch(self) -> int:
        return len(self.seqlens)

    @property
    def max_seqlen(self) -> int:
        return int(max(self.seqlens))

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


STREAM_8K = {"kind": "streaming", "sink": 128, "window": 1024}
BLOCK_32K = {"kind": "block", "block": 128, "sink_blocks": 1, "local_blocks": 8, "stride_blocks": 16}
ROUTER_4096 = {"d_model": 4096, "d_router": 64, "w_std": 0.02, "threshold": 0.0}

WORKLOADS = {
    # fp32 single layer, 512 tokens, GQA 4:1, head_dim 64, forced mask [full, streaming].
    "fp32-512-s4w64": Workload(
        name="fp32-512-s4w64", dtype="f32", seqlens=(512,), n_q_heads=8, n_kv_heads=2,
        head_dim=64, qkv_scale=1.0, qkv_seed=0,
        sparse={"kind": "streaming", "sink": 4, "window": 64}, forced_mask=((1, 0),)),
    # Llama-3-8B-shaped layer at 8K with the router; sparse heads stream 128 sink + 1024 window.
    "llama8b-8k-stream-router": Workload(
        name="llama8b-8k-stream-router", dtype="bf16", seqlens=(8192,), n_q_heads=32,
        n_kv_heads=8, head_dim=128, qkv_scale=0.5, qkv_seed=0, sparse=STREAM_8K,
        router=dict(ROUTER_4096, w_seed=0, hidden_seeds=(0,))),
    # Same layer at 32K; sparse heads use the fixed block-sparse pattern (block 128).
    "llama8b-32k-block-router": Workload(
        name="llama8b-32k-block-router", dtype="bf16", seqlens=(32768,), n_q_heads=32,
        n_kv_heads=8, head_dim=128, qkv_scale=0.5, qkv_seed=0, sparse=BLOCK_32K,
        router=dict(ROUTER_4096, w_seed=1, hidden_seeds=(1,))),
    # Qwen-style layer at 64K, 28 query / 4 KV heads (G=7), forced sparse-fraction sweep.
    "qwen-64k-stream-sweep": Workload(
        name="qwen-64k-stream-sweep", dtype="bf16", seqlens=(65536,), n_q_heads=28,
        n_kv_heads=4, head_dim=128, qkv_scale=0.5, qkv_seed=0,
        sparse={"kind": "streaming", "sink": 128, "window": 2048}, forced_mask=((0, 0, 0, 0),)),
    # Packed variable-length batch with per-sequence routing.
    "varlen-4seq-184k-stream-router": Workload(
        name="varlen-4seq-184k-stream-router", dtype="bf16",
        seqlens=(4096, 16384, 32768, 131072), n_q_heads=32, n_kv_heads=8, head_dim=128,
        qkv_scale=0.5, qkv_seed=0, sparse=STREAM_8K,
        router=dict(ROUTER_4096, w_seed=0, hidden_seeds=(10, 11, 12, 13))),
}
# Order of the configurations as the workload list states them.
WORKLOAD_ORDER = ["fp32-512-s4w64", "llama8b-8k-stream-router", "llama8b-32k-block-router",
                  "qwen-64k-stream-sweep", "varlen-4seq-184k-stream-router"]


def sweep_mask(n_kv_heads: int, sparse_fraction: float, batch: int = 1) -> np.ndarray:
    """Forced mask for a sparse-head fraction: the lowest-index KV heads are sparse."""
    k = int(round(sparse_fraction * n_kv_heads))
    row = np.ones(n_kv_heads, dtype=np.int32)
    row[:k] = 0
    return np.tile(row, (batch, 1))


def forced_mask(w: Workload) -> Optional[np.ndarray]:
    if w.forced_mask is None:
        return None
    return np.asarray(w.forced_mask, dtype=np.int32).reshape(w.batch, w.n_kv_heads)


def make_qkv(w: Workload) -> dict:
    """q [T,Hq,D], k/v [T,Hkv,D]: uint16 bf16 bit patterns, or float32 for f32 workloads."""
    T, D = w.total_tokens, w.head_dim
    shapes = {"q": (T, w.n_q_heads, D), "k": (T, w.n_kv_heads, D), "v": (T, w.n_kv_heads, D)}
    tags = {"q": TAG_Q, "k": TAG_K, "v": TAG_V}
    out = {}
    for name, shp in shapes.items():
        x = draw_f32(w.qkv_seed, tags[name], shp, w.qkv_scale)
        out[name] = round_bf16_bits(x) if w.dtype == "bf16" else x
    return out


def make_router_inputs(w: Workload, w_std: Optional[float] = None) -> dict:
    """hidden [T,d_model] bf16 bits (sequence b drawn from its own seed), w1 [d_router,d_model]
    and w2 [Hkv,d_router] in fp32.  ``w_std`` overrides the weight scale (router stress case)."""
    r = w.router
    assert r is not None, f"{w.name} has no router"
    d, dr = r["d_model"], r["d_router"]
    std = r["w_std"] if w_std is None else w_std
    parts = [draw_bf16_bits(seed, TAG_HIDDEN, (n, d)) for seed, n in zip(r["hidden_seeds"], w.seqlens)]
    hidden = parts[0] if len(parts) == 1 else np.concatenate(parts, axis=0)
    w1 = draw_f32(r["w_seed"], TAG_W1, (dr, d), std)
    w2 = draw_f32(r["w_seed"], TAG_W2, (w.n_kv_heads, dr), std)
    return {"hidden": hidden, "w1": w1, "w2": w2, "threshold": float(r["threshold"])}


def sample_rows(seqlen: int, reach: int, block: int = 128, every: int = 16) -> np.ndarray:
    """Deterministic row sample of one sequence for checks at full size: the first
    ``2*reach`` rows, every ``every``-th row block of ``block`` rows, and the last block."""
    rows = set(range(min(seqlen, 2 * reach)))
    nb = (seqlen + block - 1) // block
    for b in range(0, nb, every):
        rows.update(range(b * block, min(seqlen, (b + 1) * block)))
    rows.update(range(max(0, seqlen - block), seqlen))
    return np.array(sorted(rows), dtype=np.int64)


def spread_rows(seqlen: int, count: int, seed: int = 0) -> np.ndarray:
    """Sorted distinct rows of one sequence: a seeded uniform draw of ``count`` rows plus the
    first and the last row."""
    rng = np.random.default_rng([seed, 99])
    rows = set(rng.choice(seqlen, size=min(count, seqlen), replace=False).tolist())
    rows.update({0, seqlen - 1})
    return np.array(sorted(rows), dtype=np.int64)


def selection_lists(seed: int, batch: int, n_kv_heads: int, seqlen: int, block: int,
                    density: float, sink_blocks: int = 1) -> dict:
    """Seeded block lists shaped like the output of a content-based block selector, in CSR
    order (sequence, KV head, query block): for query block ``qb`` the first ``sink_blocks``
    blocks, the block ``qb`` itself and each earlier block with probability ``density``.
    The draw for row r uses ``default_rng([seed, 7, r])``."""
    nqb = (seqlen + block - 1) // block
    rp, ci = [0], []
    for r in range(batch * n_kv_heads * nqb):
        qb = r % nqb
        rng = np.random.default_rng([seed, 7, r])
        pick = rng.random(qb) < density
        pick[:min(sink_blocks, qb)] = True
        ci.extend(np.nonzero(pick)[0].tolist())
        ci.append(qb)
        rp.append(len(ci))
    return {"kind": "block_list", "block": block, "qblocks": nqb,
            "row_ptr": np.asarray(rp, dtype=np.int32), "col_idx": np.asarray(ci, dtype=np.int32)}

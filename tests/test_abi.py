"""C-ABI contract checks that need no GPU: the library loads, exports every declared symbol,
rejects invalid arguments on the host before any HIP call, sizes its workspaces
monotonically, and its host-side entry counter agrees with the oracle's enumeration."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from synth import inputs as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "elastic.h")

ext = pytest.importorskip("hybrid_sparse_full_elastic_amd")
if not os.path.exists(ext.LIB_PATH):
    pytest.skip("libelastic.so not built", allow_module_level=True)
L = ext.lib
FAKE = C.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(elastic_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    syms = declared_symbols()
    assert {"elastic_route", "elastic_attn_prefill", "elastic_attn_entries"} <= set(syms)
    for s in syms:
        assert hasattr(L, s), s


def test_version_and_status_strings():
    assert L.elastic_abi_version() == ext.ABI_VERSION
    for st in range(5):
        assert L.elastic_status_string(st).decode() not in ("", "unknown status")
    assert L.elastic_status_string(99).decode() == "unknown status"


def _attn(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dtype=0, cu=None, batch=1, T=256, maxlen=256, hq=8,
             hkv=2, D=128, scale=0.0, mask=None, sparse=ext.sparse_cfg({"kind": "streaming", "sink": 4, "window": 64}),
             lse=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    sp = C.byref(a["sparse"]) if a["sparse"] is not None else None
    return L.elastic_attn_prefill(a["q"], a["k"], a["v"], a["o"], a["dtype"], a["cu"], a["batch"],
                                  a["T"], a["maxlen"], a["hq"], a["hkv"], a["D"], a["scale"],
                                  a["mask"], sp, a["lse"], a["ws"], a["wsb"], a["stream"])


def test_attention_validation_without_gpu():
    EINVAL, EUNS, EWS = 1, 2, 3
    assert _attn(q=None) == EINVAL
    assert _attn(o=None) == EINVAL
    assert _attn(batch=0) == EINVAL
    assert _attn(batch=2, cu=None) == EINVAL
    assert _attn(hq=6, hkv=4) == EINVAL
    assert _attn(T=-1) == EINVAL
    assert _attn(mask=FAKE, sparse=None) == EINVAL
    assert _attn(D=96) == EUNS
    assert _attn(dtype=7) == EUNS
    assert _attn(hq=512, hkv=1) == EUNS
    assert _attn(sparse=ext.sparse_cfg({"kind": "streaming", "sink": 4, "window": 0})) == EINVAL
    assert _attn(sparse=ext.sparse_cfg({"kind": "streaming", "sink": -1, "window": 8})) == EINVAL
    bad_kind = ext.SparseCfg(9, 0, 1, 0, 0, 0, 0)
    assert _attn(sparse=bad_kind) == EINVAL
    blk = {"kind": "block", "block": 96, "sink_blocks": 1, "local_blocks": 8, "stride_blocks": 16}
    assert _attn(sparse=ext.sparse_cfg(blk)) == EUNS
    assert _attn(ws=None) == EWS
    need = ext.attn_workspace_size(0, 1, 256, 8, 2, 128)
    assert need > 0
    assert _attn(wsb=need - 1) == EWS
    assert _attn(T=0, q=None, k=None, v=None, o=None, wsb=need) == 0  # empty input: no-op


def _attn_kv(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dtype=0, cuq=None, cuk=None, batch=1, Tq=256, Tk=512,
             mq=256, mk=512, qpos=-1, kpos=0, hq=8, hkv=2, D=128, scale=0.0, mask=None,
             sparse=ext.sparse_cfg({"kind": "streaming", "sink": 4, "window": 64}), lse=None,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    sp = C.byref(a["sparse"]) if a["sparse"] is not None else None
    return L.elastic_attn_prefill_kv(a["q"], a["k"], a["v"], a["o"], a["dtype"], a["cuq"], a["cuk"],
                                     a["batch"], a["Tq"], a["Tk"], a["mq"], a["mk"], a["qpos"],
                                     a["kpos"], a["hq"], a["hkv"], a["D"], a["scale"], a["mask"], sp,
                                     a["lse"], a["ws"], a["wsb"], a["stream"])


def test_attention_kv_validation_without_gpu():
    EINVAL, EUNS, EWS = 1, 2, 3
    assert _attn_kv(kpos=32) == EINVAL            # key range must start on a 64-key tile
    assert _attn_kv(kpos=-64) == EINVAL
    assert _attn_kv(qpos=-2) == EINVAL
    assert _attn_kv(k=None) == EINVAL
    assert _attn_kv(batch=2, cuq=FAKE, cuk=None) == EINVAL
    assert _attn_kv(qpos=2 ** 31 - 100) == EINVAL  # positions past int32
    blk = {"kind": "block", "block": 128, "sink_blocks": 1, "local_blocks": 8, "stride_blocks": 16}
    assert _attn_kv(sparse=ext.sparse_cfg(blk), kpos=64) == EINVAL  # not block aligned
    assert _attn_kv(D=80) == EUNS
    assert _attn_kv(ws=None) == EWS
    need = ext.attn_workspace_size(0, 1, 256, 8, 2, 128)
    assert _attn_kv(wsb=need - 1) == EWS
    assert _attn_kv(Tq=0, q=None, o=None, wsb=need) == 0   # no query rows: no-op
    assert _attn_kv(Tk=0, k=None, v=None, Tq=0, q=None, o=None, wsb=need) == 0


def test_lse_merge_validation_without_gpu():
    EINVAL, EUNS = 1, 2
    m = L.elastic_lse_merge
    assert m(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 10, 0, 128, None) == EINVAL
    assert m(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, -1, 8, 128, None) == EINVAL
    assert m(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 10, 8, 96, None) == EUNS
    assert m(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 5, 10, 8, 128, None) == EUNS
    assert m(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 10, 8, 128, None) == EINVAL
    assert m(None, None, None, None, None, None, 0, 0, 8, 128, None) == 0  # no rows: no-op


def _route(**kw):
    a = dict(hidden=FAKE, dtype=0, cu=None, batch=1, T=1024, d=4096, ph=0, pt=0, w1=FAKE, dr=64,
             w2=FAKE, hkv=8, thr=0.0, logits=None, mask=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return L.elastic_route(a["hidden"], a["dtype"], a["cu"], a["batch"], a["T"], a["d"], a["ph"],
                           a["pt"], a["w1"], a["dr"], a["w2"], a["hkv"], a["thr"], a["logits"],
                           a["mask"], a["ws"], a["wsb"], a["stream"])


def test_route_validation_without_gpu():
    EINVAL, EUNS, EWS = 1, 2, 3
    assert _route(w1=None) == EINVAL
    assert _route(mask=None) == EINVAL
    assert _route(hidden=None) == EINVAL
    assert _route(batch=3) == EINVAL
    assert _route(ph=-1) == EINVAL
    assert _route(d=4100) == EUNS
    assert _route(dr=300) == EUNS
    assert _route(hkv=257) == EUNS
    assert _route(dtype=5) == EUNS
    assert _route(ws=None) == EWS
    need = ext.route_workspace_size(1, 1024, 4096)
    assert _route(wsb=need - 1) == EWS


def test_workspace_sizes_are_monotone():
    for dtype in (0, 1):
        prev = 0
        for T in (1, 100, 4096, 65536, 184320):
            s = ext.attn_workspace_size(dtype, 4, T, 32, 8, 128)
            assert s >= prev and s % 256 == 0
            prev = s
    prev = 0
    for T in (0, 1, 8192, 32768):
        s = ext.route_workspace_size(1, T, 4096)
        assert s >= prev
        prev = s
    assert ext.attn_workspace_size(0, 1, 100, 6, 4, 128) == 0  # heads not divisible


@pytest.mark.parametrize("sparse", [
    {"kind": "streaming", "sink": 4, "window": 64},
    {"kind": "streaming", "sink": 0, "window": 1},
    {"kind": "streaming", "sink": 128, "window": 1024},
    {"kind": "block", "block": 64, "sink_blocks": 1, "local_blocks": 2, "stride_blocks": 5},
    {"kind": "block", "block": 128, "sink_blocks": 1, "local_blocks": 8, "stride_blocks": 16},
    {"kind": "block", "block": 64, "sink_blocks": 0, "local_blocks": 0, "stride_blocks": 0},
    {"kind": "block", "block": 64, "sink_blocks": 3, "local_blocks": 1, "stride_blocks": 2},
])
def test_entry_counter_matches_oracle_enumeration(sparse):
    lens = [1, 63, 64, 65, 700, 2500]
    mask = np.array([[1, 0, 0], [0, 1, 0], [0, 0, 1], [1, 1, 0], [0, 1, 1], [1, 0, 1]])
    got = ext.attn_entries(lens, mask, 6, 3, sparse)
    assert got == oracle.entries(lens, mask, sparse, 6, 3)
    assert ext.attn_entries(lens, None, 6, 3, sparse) == oracle.entries(lens, None, sparse, 6, 3)


def test_entry_counter_at_workload_sizes():
    w = syn.WORKLOADS["llama8b-32k-block-router"]
    assert ext.attn_entries([32768], [[0]], 1, 1, w.sparse) == 68370432
    assert ext.attn_entries([32768], [[1]], 1, 1, w.sparse) == 32768 * 32769 // 2
    w = syn.WORKLOADS["qwen-64k-stream-sweep"]
    assert ext.attn_entries([65536], [[0]], 1, 1, w.sparse) == 140239936
    w = syn.WORKLOADS["fp32-512-s4w64"]
    assert ext.attn_entries([512], [[1, 0]], 8, 2, w.sparse) == 4 * (512 * 513 // 2) + 4 * 32538


def _lists(rows, B=64):
    rp, ci = [0], []
    for r in rows:
        ci.extend(r)
        rp.append(len(ci))
    return {"kind": "block_list", "block": B, "qblocks": len(rows), "row_ptr": rp, "col_idx": ci}


def test_block_list_entry_counter_matches_oracle():
    """The library's host counter for block lists (elastic_attn_entries_lists, fed host copies
    of the CSR) against the oracle's enumeration: varlen, mixed head modes, and lists with
    repeats, blocks after the query block, negative indices and empty rows."""
    rng = np.random.default_rng(5)
    lens, B, hkv, hq = [300, 0, 64, 129, 1], 64, 2, 8
    nqb = -(-max(lens) // B)
    rows = []
    for _ in range(len(lens) * hkv):
        for qb in range(nqb):
            r = rng.integers(-1, nqb + 2, size=rng.integers(0, 6)).tolist()  # repeats, later, -1
            rows.append(r)
    lists = dict(_lists(rows, B), qblocks=nqb)
    for mask in ([[0, 1], [0, 0], [1, 0], [0, 0], [0, 1]], [[0, 0]] * 5, None):
        got = ext.block_list_entries(lens, mask, hq, hkv, lists)
        assert got == oracle.entries(lens, mask, lists, hq, hkv), mask
    with pytest.raises(ValueError):                   # row pointers for too few rows
        ext.block_list_entries(lens, None, hq, hkv, dict(lists, qblocks=nqb + 1))
    # the closed-form counter declines block lists with sparse heads
    cfg = ext.SparseCfg(2, 0, 0, 64, 0, 0, 0, nqb, 0x1000, 0x1000)
    lns = (C.c_int32 * 1)(300)
    m = (C.c_int32 * 2)(0, 1)
    out = C.c_int64(0)
    assert L.elastic_attn_entries(lns, 1, m, 8, 2, C.byref(cfg), C.byref(out)) == 2


def test_block_list_entry_counter_validation():
    EINVAL, EUNS = 1, 2
    out = C.c_int64(0)
    arr = lambda *v: (C.c_int32 * len(v))(*v)  # noqa: E731
    f = L.elastic_attn_entries_lists
    rp, ci = arr(0, 1, 2, 2, 3), arr(0, 0, 1)   # 1 sequence x 1 head x 4 query blocks
    assert f(arr(200), 1, None, 4, 1, 64, 4, rp, ci, C.byref(out)) == 0
    assert out.value == 4 * (200 * 201 // 2)                                  # all heads full
    assert f(arr(200), 1, arr(0), 4, 1, 64, 4, rp, ci, C.byref(out)) == 0
    # query block 0 lists block 0, block 1 lists block 0, block 2 none, block 3 (8 rows) block 1
    assert out.value == 4 * (64 * 65 // 2 + 64 * 64 + 0 + 8 * 64)
    assert f(arr(300), 1, arr(0), 4, 1, 64, 4, rp, ci, C.byref(out)) == EINVAL  # 5 query blocks
    assert f(arr(200), 1, arr(0), 4, 1, 96, 4, rp, ci, C.byref(out)) == EUNS
    assert f(arr(200), 1, arr(0), 4, 1, 64, 4, arr(0, 2, 1, 2, 3), ci, C.byref(out)) == EINVAL
    assert f(arr(200), 1, arr(0), 4, 1, 64, 4, None, ci, C.byref(out)) == EINVAL
    assert f(arr(200), 1, arr(0), 4, 3, 64, 4, rp, ci, C.byref(out)) == EINVAL  # 4 % 3 != 0
    assert f(arr(-1), 1, arr(0), 4, 1, 64, 4, rp, ci, C.byref(out)) == EINVAL


def test_misaligned_tensors_are_rejected():
    EINVAL = 1
    odd = C.c_void_p(0x1008)
    for name in ("q", "k", "v", "o"):
        assert _attn(**{name: odd}) == EINVAL, name
    assert _attn_kv(q=odd) == EINVAL
    assert L.elastic_lse_merge(odd, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 16, 8, 128, None) == EINVAL
    assert L.elastic_lse_merge(FAKE, FAKE, FAKE, FAKE, odd, FAKE, 0, 16, 8, 128, None) == EINVAL
    assert L.elastic_route(odd, 0, None, 1, 128, 512, 0, 0, FAKE, 64, FAKE, 8, 0.0, None, FAKE,
                           FAKE, 1 << 30, None) == EINVAL


def test_attention_kernel_argument_layout():
    """The bf16 attention kernels read their argument struct through the argument-segment
    pointer at offset 0; the build checks each instance's code-object metadata for that."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_elastic_build", os.path.join(ROOT, "hybrid_sparse_full_elastic_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    obj = os.path.join(b.BUILD_DIR, "attn_bf16.o")
    if not os.path.exists(obj):
        pytest.skip("no build objects")
    meta = b.kernel_metadata(obj)
    assert b.check_attn_kernargs(meta) == 6          # D 64/128 x three sparse kinds
    bad = [dict(m) for m in meta]
    bad[0][".args"] = [{".offset": 8, ".size": 168, ".value_kind": "by_value"}]
    with pytest.raises(RuntimeError):
        b.check_attn_kernargs(bad)
    bad[0][".args"] = [{".offset": 0, ".size": 8, ".value_kind": "global_buffer"},
                       {".offset": 8, ".size": 168, ".value_kind": "by_value"}]
    with pytest.raises(RuntimeError):
        b.check_attn_kernargs(bad)


def test_block_list_validation_without_gpu():
    EINVAL, EUNS = 1, 2
    assert _attn(sparse=ext.SparseCfg(2, 0, 0, 64, 0, 0, 0, 0, 0x1000, 0x1000), mask=FAKE) == EINVAL
    assert _attn(sparse=ext.SparseCfg(2, 0, 0, 64, 0, 0, 0, 4, None, 0x1000), mask=FAKE) == EINVAL
    assert _attn(sparse=ext.SparseCfg(2, 0, 0, 96, 0, 0, 0, 4, 0x1000, 0x1000), mask=FAKE) == EUNS
    # T = 256 needs 4 query-block rows of 64 tokens: 3 are too few
    assert _attn(sparse=ext.SparseCfg(2, 0, 0, 64, 0, 0, 0, 3, 0x1000, 0x1000), mask=FAKE) == EINVAL
    # key ranges must start on a block of the list
    assert _attn_kv(sparse=ext.SparseCfg(2, 0, 0, 128, 0, 0, 0, 16, 0x1000, 0x1000), mask=FAKE,
                    kpos=64) == EINVAL


def _ret(**kw):
    a = dict(q=FAKE, k=FAKE, dtype=0, cu=None, batch=1, T=1024, ms=1024, hq=32, hkv=8, D=128,
             scale=0.0, needle=FAKE, sq=FAKE, skv=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return L.elastic_retrieval_scores(a["q"], a["k"], a["dtype"], a["cu"], a["batch"], a["T"],
                                      a["ms"], a["hq"], a["hkv"], a["D"], a["scale"], a["needle"],
                                      a["sq"], a["skv"], a["ws"], a["wsb"], a["stream"])


def test_retrieval_and_assignment_validation_without_gpu():
    EINVAL, EUNS, EWS = 1, 2, 3
    assert _ret(needle=None) == EINVAL
    assert _ret(sq=None, skv=None) == EINVAL
    assert _ret(q=None) == EINVAL
    assert _ret(hq=30) == EINVAL                      # not a multiple of n_kv_heads
    assert _ret(batch=2) == EINVAL                    # several sequences need cu_seqlens
    assert _ret(T=2048) == EINVAL                     # one sequence longer than max_seqlen
    assert _ret(q=C.c_void_p(0x1008)) == EINVAL      # 16-byte alignment
    assert _ret(D=96) == EUNS
    assert _ret(dtype=7) == EUNS
    assert _ret(ws=None) == EWS
    need = ext.retrieval_workspace_size(1, 1024, 32)
    assert need > 0 and _ret(wsb=need - 1) == EWS
    assert _ret(batch=0, q=None, k=None, needle=None) == 0   # nothing to score
    a = L.elastic_static_assignment
    assert a(FAKE, 8, -0.1, FAKE, None) == EINVAL
    assert a(FAKE, 8, 1.5, FAKE, None) == EINVAL
    assert a(FAKE, -1, 0.5, FAKE, None) == EINVAL
    assert a(None, 8, 0.5, FAKE, None) == EINVAL
    assert a(FAKE, 16385, 0.5, FAKE, None) == EUNS
    assert a(None, 0, 0.5, None, None) == 0                  # no units: no-op


def _noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dtype=0, cu=None, batch=1, T=256, maxlen=256, hq=8,
             hkv=2, D=128, scale=0.0, mask=None, sparse=ext.sparse_cfg({"kind": "streaming", "sink": 4, "window": 64}),
             lse=None, stream=None)
    a.update(kw)
    sp = C.byref(a["sparse"]) if a["sparse"] is not None else None
    return L.elastic_attn_prefill_noalloc(a["q"], a["k"], a["v"], a["o"], a["dtype"], a["cu"],
                                          a["batch"], a["T"], a["maxlen"], a["hq"], a["hkv"], a["D"],
                                          a["scale"], a["mask"], sp, a["lse"], a["stream"])


def test_noalloc_validation_without_gpu():
    """The allocation-free variant validates on the host, and rejects problems whose scheduler
    scratch exceeds the library's fixed array, before any HIP call."""
    EINVAL, EUNS, EWS = 1, 2, 3
    assert _noalloc(q=None) == EINVAL
    assert _noalloc(o=C.c_void_p(0x1008)) == EINVAL
    assert _noalloc(hq=6, hkv=4) == EINVAL
    assert _noalloc(D=96) == EUNS
    assert _noalloc(T=0, maxlen=0) == 0                      # nothing to do, no HIP call
    limit = 8 << 20
    big = 4_000_000                                          # 500,000 items of 32 / 8 heads
    assert ext.attn_workspace_size(0, 1, big, 32, 8, 128) > limit
    assert _noalloc(T=big, maxlen=big, hq=32, hkv=8) == EWS
    msg = L.elastic_last_error().decode()
    assert "scratch" in msg and str(limit) in msg, msg
    ok = 3_000_000
    assert ext.attn_workspace_size(0, 1, ok, 32, 8, 128) <= limit

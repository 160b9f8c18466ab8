"""GPU parity of the deployment forms against the fp64 oracle, through the C ABI: chunked
prefill (queries against their whole prefix, bottom-right aligned), key-range splits merged
by LSE, the LSE-merge kernel on its own, and block-granular streaming ("Elastic Attention",
arXiv 2601.17367; paperlayer summary, appendix D.1 "Sparse Inference": block 64, chunk
16,384, 128 sink tokens).

Small cases compare every element, including rows that see no key of a range (o = 0,
lse = -inf).  At 32K, chunked prefill with chunk 16,384 must reproduce the unchunked launch
bit for bit (same query tiles, same key tiles in the same order), and sampled rows are
checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from synth import inputs as syn
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

ext = None


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    global ext
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import hybrid_sparse_full_elastic_amd as m  # no fallback: must load the HIP library
    ext = m
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


STREAM = {"kind": "streaming", "sink": 16, "window": 100}
BLOCK = {"kind": "block", "block": 64, "sink_blocks": 1, "local_blocks": 2, "stride_blocks": 3}
BSTREAM = oracle.block_streaming(128, 256, 64)
CASES = [
    # name, seqlens, hq, hkv, D, sparse, mask
    ("stream-g4-d128", [600], 8, 2, 128, STREAM, [[1, 0]]),
    ("block-g4-d64", [517], 8, 2, 64, BLOCK, [[0, 1]]),
    ("bstream-g7-d128", [450], 14, 2, 128, BSTREAM, [[0, 1]]),
    ("full-g8-d128", [333], 8, 1, 128, None, None),
    # large GQA ratios: items of 8 and of one query token
    ("stream-g32-d128", [300], 64, 2, 128, STREAM, [[0, 1]]),
    ("block-g256-d64", [150], 256, 1, 64, BLOCK, [[0]]),
]


def _draw(seed, T, hq, hkv, D, dtype="bf16", scale=0.5):
    draw = syn.draw_bf16_bits if dtype == "bf16" else syn.draw_f32
    return {"q": draw(seed, 0, (T, hq, D), scale), "k": draw(seed, 1, (T, hkv, D), scale),
            "v": draw(seed, 2, (T, hkv, D), scale)}


def _cu(lens):
    return torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=H.DEV)


def _mask(m):
    return None if m is None else torch.tensor(np.asarray(m), dtype=torch.int32, device=H.DEV)


def _kv_call(q, k, v, cu_q, cu_k, mask, sparse, q_pos=-1, k_pos=0, lse=True):
    Tq, hq, _ = q.shape
    l = torch.full((hq, Tq), float("nan"), dtype=torch.float32, device=H.DEV) if lse else None
    o = ext.attn_prefill_kv(q, k, v, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, q_pos=q_pos,
                            k_pos=k_pos, head_mask=mask, sparse=sparse, lse=l)
    return o, l


def _check(o, l, ro, rl, what, dtype):
    o, l = H.to_f64(o), H.to_f64(l)
    if dtype == "bf16":
        H.assert_bf16_close(o, ro, what)
        atol = H.BF16_LSE_ATOL
    else:
        H.assert_f32_close(o, ro, what)
        atol = 1e-5
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(l), ~fin), what          # empty rows: lse = -inf
    np.testing.assert_allclose(l[fin], rl[fin], rtol=0, atol=atol)
    assert np.all(o[np.transpose(~fin)] == 0), what            # empty rows: o = 0


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("chunk", [128, 200])
def test_chunked_prefill_every_element(case, chunk):
    name, seqlens, hq, hkv, D, sparse, mask = case
    print(f"[case] chunked {name} chunk={chunk}", flush=True)
    n = seqlens[0]
    data = _draw(21, n, hq, hkv, D)
    q, k, v = H.to_dev(data["q"]), H.to_dev(data["k"]), H.to_dev(data["v"])
    m = _mask(mask)
    o = torch.empty_like(q)
    lse = torch.empty((hq, n), dtype=torch.float32, device=H.DEV)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        oc, lc = _kv_call(q[c0:c1], k[:c1], v[:c1], None, None, m, sparse)
        o[c0:c1] = oc
        lse[:, c0:c1] = lc
    torch.cuda.synchronize()
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], None, mask, sparse)
    _check(o, lse, ro, rl, f"chunked {name}", "bf16")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_keys_partials_and_merge(case):
    """Each partial matches the oracle's key-range attention (empty rows included), and the
    merge kernel's result matches attention over all keys."""
    name, seqlens, hq, hkv, D, sparse, mask = case
    print(f"[case] split {name}", flush=True)
    n = seqlens[0]
    data = _draw(22, n, hq, hkv, D)
    q, k, v = H.to_dev(data["q"]), H.to_dev(data["k"]), H.to_dev(data["v"])
    m = _mask(mask)
    cut = 192 if sparse is None or sparse.get("block", 64) == 64 else 256
    oa, la = _kv_call(q, k[:cut], v[:cut], None, None, m, sparse, q_pos=0, k_pos=0)
    ob, lb = _kv_call(q, k[cut:], v[cut:], None, None, m, sparse, q_pos=0, k_pos=cut)
    torch.cuda.synchronize()
    ra, rla = oracle.attention_kv(data["q"], data["k"][:cut], data["v"][:cut], None, None, mask,
                                  sparse, q_pos=[0], k_pos=0)
    rb, rlb = oracle.attention_kv(data["q"], data["k"][cut:], data["v"][cut:], None, None, mask,
                                  sparse, q_pos=[0], k_pos=cut)
    _check(oa, la, ra, rla, f"part A {name}", "bf16")
    _check(ob, lb, rb, rlb, f"part B {name}", "bf16")
    om, lm = ext.lse_merge(oa, la, ob, lb)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], None, mask, sparse)
    _check(om, lm, ro, rl, f"merged {name}", "bf16")


def test_fp32_chunks_and_merge():
    n, D = 300, 64
    data = _draw(23, n, 8, 2, D, dtype="f32", scale=1.0)
    q, k, v = H.to_dev(data["q"]), H.to_dev(data["k"]), H.to_dev(data["v"])
    mask = [[0, 1]]
    m = _mask(mask)
    o = torch.empty_like(q)
    lse = torch.empty((8, n), dtype=torch.float32, device=H.DEV)
    for c0 in range(0, n, 96):
        c1 = min(n, c0 + 96)
        o[c0:c1], lse[:, c0:c1] = _kv_call(q[c0:c1], k[:c1], v[:c1], None, None, m, BLOCK)
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], None, mask, BLOCK)
    _check(o, lse, ro, rl, "fp32 chunked", "f32")
    oa, la = _kv_call(q, k[:128], v[:128], None, None, m, BLOCK, q_pos=0, k_pos=0)
    ob, lb = _kv_call(q, k[128:], v[128:], None, None, m, BLOCK, q_pos=0, k_pos=128)
    om, lm = ext.lse_merge(oa, la, ob, lb, out=oa, lse_out=la)  # in place
    torch.cuda.synchronize()
    _check(om, lm, ro, rl, "fp32 merged in place", "f32")


def test_varlen_chunk_per_sequence_bottom_right():
    """One call per chunk index over a packed batch: sequence b contributes its chunk rows as
    queries and its prefix up to the chunk end as keys (bottom-right per sequence)."""
    lens = [300, 1, 0, 450, 129]
    hq, hkv, D, chunk = 8, 2, 128, 128
    T = sum(lens)
    data = _draw(24, T, hq, hkv, D)
    mask = [[1, 0], [0, 1], [1, 1], [0, 0], [0, 1]]
    cu = np.concatenate([[0], np.cumsum(lens)])
    qd, kd, vd = H.to_dev(data["q"]), H.to_dev(data["k"]), H.to_dev(data["v"])
    o = torch.zeros_like(qd)
    lse = torch.zeros((hq, T), dtype=torch.float32, device=H.DEV)
    for c0 in range(0, max(lens), chunk):
        qi = [np.arange(cu[b] + min(c0, n), cu[b] + min(c0 + chunk, n)) for b, n in enumerate(lens)]
        ki = [np.arange(cu[b], cu[b] + min(c0 + chunk, n)) for b, n in enumerate(lens)]
        qrows, krows = np.concatenate(qi), np.concatenate(ki)
        cq, ck = _cu([len(x) for x in qi]), _cu([len(x) for x in ki])
        qr = torch.from_numpy(qrows).to(H.DEV)
        kr = torch.from_numpy(krows).to(H.DEV)
        oc, lc = _kv_call(qd[qr].contiguous(), kd[kr].contiguous(), vd[kr].contiguous(), cq, ck,
                          _mask(mask), STREAM)
        o[qr] = oc
        lse[:, qr] = lc
    torch.cuda.synchronize()
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], cu, mask, STREAM)
    _check(o, lse, ro, rl, "varlen chunked", "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lse_merge_kernel(dtype):
    rows, heads, D = 777, 6, 128
    rng = np.random.default_rng(25)
    oa = rng.standard_normal((rows, heads, D)).astype(np.float32)
    ob = rng.standard_normal((rows, heads, D)).astype(np.float32)
    la = (rng.standard_normal((heads, rows)) * 4).astype(np.float32)
    lb = (rng.standard_normal((heads, rows)) * 4).astype(np.float32)
    la[0, :50] = -np.inf               # one side empty
    lb[1, 10:20] = -np.inf
    la[2, 30:40] = lb[2, 30:40] = -np.inf  # both empty
    oa[30:40, 2] = ob[30:40, 2] = 0.0
    if dtype == "bf16":
        oa_bits, ob_bits = syn.round_bf16_bits(oa), syn.round_bf16_bits(ob)
        ta, tb = H.to_dev(oa_bits), H.to_dev(ob_bits)
        ra_in, rb_in = oracle.decode_bf16(oa_bits), oracle.decode_bf16(ob_bits)
    else:
        ta, tb = H.to_dev(oa), H.to_dev(ob)
        ra_in, rb_in = oa.astype(np.float64), ob.astype(np.float64)
    om, lm = ext.lse_merge(ta, H.to_dev(la), tb, H.to_dev(lb))
    torch.cuda.synchronize()
    ro, rl = oracle.lse_merge(ra_in, la, rb_in, lb)
    got, gl = H.to_f64(om), H.to_f64(lm)
    tol = 2 ** -8 * np.abs(ro) + 1e-6 if dtype == "bf16" else 1e-5 * np.abs(ro) + 1e-6
    assert np.all(np.abs(got - ro) <= tol)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(gl), ~fin)
    np.testing.assert_allclose(gl[fin], rl[fin], rtol=0, atol=1e-5)


# ------------------------------------------------------------------ full size (32K layer)
@pytest.fixture(scope="module")
def layer32k():
    w = syn.WORKLOADS["llama8b-32k-block-router"]
    data, q, k, v = H.qkv_dev(w)
    return w, data, q, k, v


def test_chunked_prefill_32k_bitwise_and_oracle(layer32k):
    """Chunk 16,384: both chunks reproduce the unchunked launch exactly; sampled rows of the
    second chunk match the oracle."""
    w, data, q, k, v = layer32k
    n, hq = q.shape[0], q.shape[1]
    mask = _mask([[1, 0, 1, 1, 0, 0, 1, 0]])
    lse_full = torch.empty((hq, n), dtype=torch.float32, device=H.DEV)
    o_full = ext.attn_prefill(q, k, v, max_seqlen=n, head_mask=mask, sparse=w.sparse, lse=lse_full)
    o = torch.empty_like(q)
    lse = torch.empty_like(lse_full)
    C = 16384
    for c0 in range(0, n, C):
        o[c0:c0 + C], lse[:, c0:c0 + C] = _kv_call(q[c0:c0 + C], k[:c0 + C], v[:c0 + C], None, None,
                                                   mask, w.sparse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_full.view(torch.int16))
    assert torch.equal(lse, lse_full)
    rows = np.sort(np.concatenate([syn.spread_rows(C, 24, 31) + C, [C, C + 1, n - 1]]))
    rows = np.unique(rows)
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], None, mask.cpu().numpy(), w.sparse,
                              rows=rows, workers=16)
    H.assert_bf16_close(H.to_f64(o[torch.from_numpy(rows).to(H.DEV)]), ro, "32K chunk 2 vs oracle")


def test_split_keys_merge_32k(layer32k):
    """Keys split at 16,384 and merged by LSE agree with the single launch and the oracle."""
    w, data, q, k, v = layer32k
    n, hq = q.shape[0], q.shape[1]
    mask = _mask([[1, 1, 0, 1, 0, 1, 0, 0]])
    C = 16384
    oa, la = _kv_call(q, k[:C], v[:C], None, None, mask, w.sparse, q_pos=0, k_pos=0)
    ob, lb = _kv_call(q, k[C:], v[C:], None, None, mask, w.sparse, q_pos=0, k_pos=C)
    om, lm = ext.lse_merge(oa, la, ob, lb)
    lse_full = torch.empty((hq, n), dtype=torch.float32, device=H.DEV)
    o_full = ext.attn_prefill(q, k, v, max_seqlen=n, head_mask=mask, sparse=w.sparse, lse=lse_full)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(lb[:, :C]))  # the first half's queries see no key of [C, n)
    H.assert_bf16_close(H.to_f64(om), H.to_f64(o_full), "32K merged vs single launch")
    assert float((lm - lse_full).abs().max()) < 1e-3
    rows = np.unique(np.concatenate([syn.spread_rows(n, 24, 32), [C - 1, C, C + 5]]))
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], None, mask.cpu().numpy(), w.sparse,
                              rows=rows, workers=16)
    H.assert_bf16_close(H.to_f64(om[torch.from_numpy(rows).to(H.DEV)]), ro, "32K merged vs oracle")


def test_block_streaming_32k(layer32k):
    """Block-granular streaming (block 64, 128 sink tokens, window 1024) on every head."""
    w, data, q, k, v = layer32k
    n, hq = q.shape[0], q.shape[1]
    sparse = oracle.block_streaming(128, 1024, 64)
    zeros = [[0] * 8]
    lse = torch.empty((hq, n), dtype=torch.float32, device=H.DEV)
    o = ext.attn_prefill(q, k, v, max_seqlen=n, head_mask=_mask(zeros), sparse=sparse, lse=lse)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([syn.spread_rows(n, 40, 33), [127, 128, 1023, 1024, 1087]]))
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], None, zeros, sparse, rows=rows,
                              workers=16)
    H.assert_bf16_close(H.to_f64(o[torch.from_numpy(rows).to(H.DEV)]), ro, "32K block streaming")
    np.testing.assert_allclose(H.to_f64(lse)[:, rows], rl, rtol=0, atol=H.BF16_LSE_ATOL)

"""Pins of the oracle's deployment forms: key-range attention, LSE merge, chunked prefill and
block-granular streaming ("Elastic Attention", arXiv 2601.17367; paperlayer summary,
appendix D.1 "Sparse Inference": block 64, chunk 16,384, 128 sink tokens).

Each check ties the new oracle functions to something outside them: the whole-sequence
oracle attention (a separate code path on local positions), brute force with Python loops on
tiny inputs, closed-form key counts, and identities of the merge."""
import math

import numpy as np
import pytest

from oracle import elastic_oracle as O

STREAM = {"kind": "streaming", "sink": 5, "window": 23}
BLOCK = {"kind": "block", "block": 16, "sink_blocks": 1, "local_blocks": 2, "stride_blocks": 4}
PATTERNS = [("full", None, None), ("stream", STREAM, [[0, 0]]), ("block", BLOCK, [[0, 0]]),
            ("mixed", STREAM, [[1, 0]])]


def _qkv(n, hq=4, hkv=2, d=16, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, hq, d)), rng.standard_normal((n, hkv, d)),
            rng.standard_normal((n, hkv, d)))


@pytest.mark.parametrize("name,sparse,mask", PATTERNS)
@pytest.mark.parametrize("cuts", [(128,), (50, 177), (1, 299)])
def test_split_keys_merge_equals_whole(name, sparse, mask, cuts):
    """P11: attending key ranges separately and merging by LSE equals attending once."""
    n = 300
    q, k, v = _qkv(n)
    o, lse = O.attention(q, k, v, None, mask, sparse)
    bounds = [0, *cuts, n]
    om, lm = None, None
    for a, b in zip(bounds[:-1], bounds[1:]):
        op, lp = O.attention_kv(q, k[a:b], v[a:b], None, None, mask, sparse, q_pos=[0], k_pos=a)
        om, lm = (op, lp) if om is None else O.lse_merge(om, lm, op, lp)
    assert np.allclose(om, o, rtol=0, atol=1e-12)
    assert np.allclose(lm, lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name,sparse,mask", PATTERNS)
@pytest.mark.parametrize("chunk", [64, 100, 299, 1000])
def test_chunked_prefill_equals_whole(name, sparse, mask, chunk):
    n = 300
    q, k, v = _qkv(n, seed=1)
    o, lse = O.attention(q, k, v, None, mask, sparse)
    oc, lc = O.chunked_prefill(q, k, v, None, mask, sparse, chunk)
    assert np.allclose(oc, o, rtol=0, atol=1e-12)
    assert np.allclose(lc, lse, rtol=0, atol=1e-12)


def test_chunked_prefill_varlen():
    lens = [70, 1, 0, 130]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = _qkv(int(cu[-1]), seed=2)
    mask = [[1, 0], [0, 1], [1, 1], [0, 0]]
    o, lse = O.attention(q, k, v, cu, mask, STREAM)
    oc, lc = O.chunked_prefill(q, k, v, cu, mask, STREAM, 48)
    assert np.allclose(oc, o, rtol=0, atol=1e-12)
    assert np.allclose(lc, lse, rtol=0, atol=1e-12)


def _brute(qv, kv, vv, qp, kp, full, sparse, scale):
    """One query row, pure Python: softmax over the allowed absolute key positions."""
    ss, vs = [], []
    for j, kj in enumerate(kv):
        if bool(O.allowed(qp, kp + j, full, sparse)):
            ss.append(scale * sum(a * b for a, b in zip(qv, kj)))
            vs.append(vv[j])
    if not ss:
        return [0.0] * len(vv[0]), -math.inf
    m = max(ss)
    w = [math.exp(s - m) for s in ss]
    tot = sum(w)
    out = [sum(wi * x[dd] for wi, x in zip(w, vs)) / tot for dd in range(len(vv[0]))]
    return out, m + math.log(tot)


@pytest.mark.parametrize("sparse,full", [(None, True), ({"kind": "streaming", "sink": 2, "window": 3}, False),
                                         ({"kind": "block", "block": 4, "sink_blocks": 1,
                                           "local_blocks": 0, "stride_blocks": 0}, False)])
def test_attention_kv_brute_force(sparse, full):
    rng = np.random.default_rng(3)
    nq, nk, d = 5, 8, 3
    q = rng.standard_normal((nq, 1, d))
    k = rng.standard_normal((nk, 1, d))
    v = rng.standard_normal((nk, 1, d))
    mask = None if full else [[0]]
    for q_pos, k_pos in ((9, 4), (4, 4), (2, 8), (0, 0)):
        o, lse = O.attention_kv(q, k, v, None, None, mask, sparse, q_pos=[q_pos], k_pos=k_pos)
        for t in range(nq):
            ob, lb = _brute(q[t, 0], k[:, 0], v[:, 0], q_pos + t, k_pos, full, sparse, d ** -0.5)
            assert np.allclose(o[t, 0], ob, rtol=0, atol=1e-13)
            assert (lse[0, t] == lb == -math.inf) or abs(lse[0, t] - lb) < 1e-13


def test_bottom_right_default():
    """q_pos None places the queries at the last key positions."""
    q, k, v = _qkv(90, seed=4)
    o1, l1 = O.attention_kv(q[60:], k, v, None, None, None, STREAM)
    o2, l2 = O.attention_kv(q[60:], k, v, None, None, None, STREAM, q_pos=[60])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o, lse = O.attention(q, k, v, None, None, STREAM)
    assert np.allclose(o1, o[60:], atol=1e-12) and np.allclose(l1, lse[:, 60:], atol=1e-12)


def test_rows_without_keys_and_merge_identity():
    q, k, v = _qkv(40, seed=5)
    # keys at positions 100.. are all in the future of queries at 0..39
    oe, le = O.attention_kv(q, k, v, None, None, None, None, q_pos=[0], k_pos=100)
    assert np.all(oe == 0) and np.all(np.isneginf(le))
    o, lse = O.attention(q, k, v, None, None, None)
    om, lm = O.lse_merge(o, lse, oe, le)
    assert np.array_equal(om, o) and np.array_equal(lm, lse)
    om, lm = O.lse_merge(oe, le, oe, le)
    assert np.all(om == 0) and np.all(np.isneginf(lm))


def test_merge_symmetric_and_disjoint_singletons():
    """Two one-key partials merge to the two-key softmax (computed by the whole-sequence path)."""
    q, k, v = _qkv(2, hq=1, hkv=1, seed=6)
    oa, la = O.attention_kv(q[1:], k[:1], v[:1], None, None, None, None, q_pos=[1], k_pos=0)
    ob, lb = O.attention_kv(q[1:], k[1:], v[1:], None, None, None, None, q_pos=[1], k_pos=1)
    o1, l1 = O.lse_merge(oa, la, ob, lb)
    o2, l2 = O.lse_merge(ob, lb, oa, la)
    assert np.allclose(o1, o2, atol=1e-15) and np.allclose(l1, l2, atol=1e-15)
    o, lse = O.attention(q, k, v, None, None, None)
    assert np.allclose(o1, o[1:], atol=1e-13) and np.allclose(l1, lse[:, 1:], atol=1e-13)


@pytest.mark.parametrize("window", [64, 512, 1024, 2048])
def test_block_streaming_counts_closed_form(window):
    """|A(i)| = keys of the window blocks up to i, plus the 128 sink tokens below them."""
    cfg = O.block_streaming(128, window, 64)
    assert cfg == {"kind": "block", "block": 64, "sink_blocks": 2,
                   "local_blocks": window // 64 - 1, "stride_blocks": 0}
    n = 3 * window + 500
    got = O.row_key_counts(n, False, cfg)
    i = np.arange(n)
    ws = np.maximum(0, (i // 64 - (window // 64 - 1)) * 64)
    want = (i - ws + 1) + np.minimum(128, ws)
    assert np.array_equal(got, want)


def test_block_streaming_32k_total():
    """Entries per query head of the 32K layer with block streaming (128 sinks, window 1024)."""
    n, w = 32768, 1024
    i = np.arange(n)
    ws = np.maximum(0, (i // 64 - (w // 64 - 1)) * 64)
    want = int(((i - ws + 1) + np.minimum(128, ws)).sum())
    assert O.entries([n], [[0]], O.block_streaming(128, w), 1, 1) == want
    # between the token-exact windows of 1024 - 63 and 1024 keys plus the sinks
    lo = O.entries([n], [[0]], {"kind": "streaming", "sink": 128, "window": w - 63}, 1, 1)
    hi = O.entries([n], [[0]], {"kind": "streaming", "sink": 128, "window": w}, 1, 1)
    assert lo <= want <= hi

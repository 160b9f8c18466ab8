"""Pins of the fp64 oracle against facts fixed by the method's definition and by mathematics.

Each test would fail for a plausible mistake in the oracle: a dropped mask term, an
off-by-one in the window or block boundaries, a wrong GQA index, a wrong softmax
normalisation or LSE, a router sign or threshold-direction error.
Source passages: paperlayer.ai summary of arXiv 2601.17367, section 2 "Hybrid Head
Mechanism" and "Sparsity Ratio Computation", section 3 "Attention Router" and
"Router Optimization", appendix C.1 (needle probing), appendix D.1 "Sparse Inference".
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import inputs as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
STREAM = {"kind": "streaming", "sink": 4, "window": 16}
BLOCK = {"kind": "block", "block": 8, "sink_blocks": 1, "local_blocks": 2, "stride_blocks": 4}


def _rand(seed, shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------------------- hand-worked examples
def test_router_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))["router"]
    for exact in (False, True):
        r = oracle.route(np.array(g["hidden"]), [0, 2], np.array(g["w1"]), np.array(g["w2"]),
                         g["threshold"], exact=exact)
        np.testing.assert_array_equal(r["mask"][0], g["mask"])
    np.testing.assert_array_equal(r["pooled"][0], g["pooled"])
    np.testing.assert_array_equal(r["z"][0], g["z"])
    np.testing.assert_array_equal(r["logits"][0], g["logits"])
    np.testing.assert_array_equal(r["mask"][0], g["mask"])


def test_attention_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))["attention"]
    q = np.array(g["q"]).reshape(3, 1, 1)
    k = np.log(np.array(g["k_logs"], dtype=np.float64)).reshape(3, 1, 1)
    v = np.array(g["v"]).reshape(3, 1, 1)
    o, lse = oracle.attention(q, k, v, None, [[1]], None, scale=1.0)
    np.testing.assert_allclose(o[:, 0, 0], g["full_o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(np.exp(lse[0]), g["full_lse_exp"], rtol=1e-13)
    for sp in ({"kind": "streaming", "sink": 1, "window": 1},
               {"kind": "block", "block": 1, "sink_blocks": 1, "local_blocks": 0, "stride_blocks": 0}):
        o, lse = oracle.attention(q, k, v, None, [[0]], sp, scale=1.0)
        np.testing.assert_allclose(o[:, 0, 0], g["stream_s1_w1_o"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(np.exp(lse[0]), g["stream_s1_w1_lse_exp"], rtol=1e-13)


# --------------------------------------------------------------------------- P1: full == dense causal
def _dense_causal(q, k, v, scale):
    """Independent dense softmax attention with -inf above the diagonal (one head)."""
    n = q.shape[0]
    s = scale * q @ k.T
    s[np.triu(np.ones((n, n), dtype=bool), 1)] = -np.inf
    s = s - s.max(1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(1, keepdims=True)
    return p @ v


def test_full_mask_equals_dense_causal_and_sdpa():
    n, Hq, Hkv, D = 200, 6, 2, 16
    q, k, v = _rand(1, (n, Hq, D)), _rand(2, (n, Hkv, D)), _rand(3, (n, Hkv, D))
    o, _ = oracle.attention(q, k, v, None, [[1, 1]], STREAM, block_rows=37)
    o_none, _ = oracle.attention(q, k, v, None, None, STREAM, block_rows=37)
    np.testing.assert_array_equal(o, o_none)
    G = Hq // Hkv
    for h in range(Hq):
        ref = _dense_causal(q[:, h], k[:, h // G], v[:, h // G], D ** -0.5)
        np.testing.assert_allclose(o[:, h], ref, rtol=0, atol=1e-12)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- P2: probabilities
@pytest.mark.parametrize("full,sparse", [(True, None), (False, STREAM), (False, BLOCK)])
def test_rows_are_distributions_on_the_allowed_set(full, sparse):
    """With v_j = e_j the output row is the probability vector itself."""
    n = 48
    q, k = _rand(4, (n, 1, 8)), _rand(5, (n, 1, 8))
    v = np.eye(n).reshape(n, 1, n)
    o, _ = oracle.attention(q, k, v, None, [[1 if full else 0]], sparse)
    p = o[:, 0, :]
    assert np.all(np.abs(p.sum(1) - 1.0) <= 1e-12)
    for i in range(n):
        for j in range(n):
            in_set = j <= i and (full or _in_set_by_hand(i, j, sparse))
            assert (p[i, j] > 0) == in_set, (i, j)


def _in_set_by_hand(i, j, sp):
    if sp["kind"] == "streaming":
        return j < sp["sink"] or j > i - sp["window"]
    B = sp["block"]
    qb, kb = i // B, j // B
    return kb < sp["sink_blocks"] or kb >= qb - sp["local_blocks"] or \
        (sp["stride_blocks"] > 0 and kb % sp["stride_blocks"] == 0)


# --------------------------------------------------------------------------- P3: key counts
def _block_count_closed_form(i, B, sinkb, local, stride):
    qb = i // B
    earlier = set(range(min(sinkb, qb))) | set(range(max(0, qb - local), qb))
    if stride > 0:
        earlier |= set(range(0, qb, stride))
    return len(earlier) * B + (i % B) + 1


@pytest.mark.parametrize("S,W", [(4, 16), (0, 1), (1, 1), (128, 1024), (7, 300)])
def test_streaming_counts_closed_form(S, W):
    n = 1500
    c = oracle.row_key_counts(n, False, {"kind": "streaming", "sink": S, "window": W})
    np.testing.assert_array_equal(c, np.minimum(np.arange(n) + 1, S + W))


@pytest.mark.parametrize("B,sinkb,local,stride", [(8, 1, 2, 4), (128, 1, 8, 16), (64, 2, 3, 0), (16, 0, 0, 5)])
def test_block_counts_closed_form(B, sinkb, local, stride):
    n = 40 * B + 5
    sp = {"kind": "block", "block": B, "sink_blocks": sinkb, "local_blocks": local, "stride_blocks": stride}
    c = oracle.row_key_counts(n, False, sp)
    ref = [_block_count_closed_form(i, B, sinkb, local, stride) for i in range(n)]
    np.testing.assert_array_equal(c, ref)


def test_workload_entry_totals():
    """Per-query-head totals of the five workloads' sparse patterns, by closed form:
    streaming sum_i min(i+1, S+W) = c(c+1)/2 + (n-c)c with c = S+W."""
    def stream_total(n, S, W):
        c = min(n, S + W)
        return c * (c + 1) // 2 + (n - c) * c
    assert stream_total(512, 4, 64) == 32538
    assert stream_total(8192, 128, 1024) == 8774208
    assert stream_total(65536, 128, 2048) == 140239936
    w = syn.WORKLOADS
    for name, n in (("fp32-512-s4w64", 512), ("llama8b-8k-stream-router", 8192)):
        sp = w[name].sparse
        assert oracle.entries([n], [[0]], sp, 1, 1) == stream_total(n, sp["sink"], sp["window"])
    # block pattern at 32K (block 128, sink 1, local 8, stride 16): sum of the closed form
    sp = w["llama8b-32k-block-router"].sparse
    n = 32768
    nb = n // 128
    tot = 0
    for qb in range(nb):
        e = _block_count_closed_form(qb * 128, 128, 1, 8, 16) - 1
        tot += 128 * e + 128 * 129 // 2
    assert tot == 68370432
    assert oracle.entries([n], [[0]], sp, 1, 1) == tot
    assert oracle.entries([n], [[1]], sp, 1, 1) == n * (n + 1) // 2


# --------------------------------------------------------------------------- P4: reductions to full
def test_special_cases_reduce_to_full():
    n, D = 130, 8
    q, k, v = _rand(6, (n, 2, D)), _rand(7, (n, 1, D)), _rand(8, (n, 1, D))
    full, lf = oracle.attention(q, k, v, None, [[1]], None)
    for sp in ({"kind": "streaming", "sink": 0, "window": n},
               {"kind": "streaming", "sink": n, "window": 1},
               {"kind": "block", "block": 8, "sink_blocks": 0, "local_blocks": 17, "stride_blocks": 0},
               {"kind": "block", "block": 8, "sink_blocks": 0, "local_blocks": 0, "stride_blocks": 1}):
        o, l = oracle.attention(q, k, v, None, [[0]], sp)
        np.testing.assert_array_equal(o, full)
        np.testing.assert_array_equal(l, lf)
    o, _ = oracle.attention(q, k, v, None, [[0]], {"kind": "streaming", "sink": 0, "window": n - 1})
    assert not np.array_equal(o, full)


# --------------------------------------------------------------------------- P5: brute force
def _brute(q, k, v, mask_row, sparse, scale):
    """Pure-Python loops: per row, fsum-normalised softmax over the allowed keys."""
    n, Hq, D = q.shape
    G = Hq // k.shape[1]
    o = [[[0.0] * D for _ in range(Hq)] for _ in range(n)]
    lse = [[0.0] * n for _ in range(Hq)]
    for h in range(Hq):
        g = h // G
        for i in range(n):
            keys = [j for j in range(i + 1) if mask_row[g] or _in_set_by_hand(i, j, sparse)]
            s = [scale * math.fsum(q[i, h, d] * k[j, g, d] for d in range(D)) for j in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            for d in range(D):
                o[i][h][d] = math.fsum(e[t] * v[keys[t], g, d] for t in range(len(keys))) / z
            lse[h][i] = m + math.log(z)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("sparse", [{"kind": "streaming", "sink": 3, "window": 5}, BLOCK])
def test_brute_force_tiny(sparse):
    n, Hq, Hkv, D = 41, 4, 2, 8
    q, k, v = _rand(9, (n, Hq, D)), _rand(10, (n, Hkv, D)), _rand(11, (n, Hkv, D))
    mrow = [1, 0]
    o, lse = oracle.attention(q, k, v, None, [mrow], sparse, block_rows=16)
    ob, lb = _brute(q, k, v, mrow, sparse, D ** -0.5)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


def test_varlen_sequences_are_independent():
    lens = [17, 1, 40]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v = _rand(12, (T, 4, 8)), _rand(13, (T, 2, 8)), _rand(14, (T, 2, 8))
    mask = np.array([[1, 0], [0, 1], [0, 0]])
    sp = {"kind": "streaming", "sink": 2, "window": 5}
    o, lse = oracle.attention(q, k, v, cu, mask, sp)
    for b in range(3):
        sl = slice(cu[b], cu[b + 1])
        ob, lb = oracle.attention(q[sl], k[sl], v[sl], None, mask[b:b + 1], sp)
        np.testing.assert_array_equal(o[sl], ob)
        np.testing.assert_array_equal(lse[:, sl], lb)
    # row subsets agree with the full evaluation
    rows = np.array([0, 16, 17, 30, 57])
    osub, lsub = oracle.attention(q, k, v, cu, mask, sp, rows=rows, heads=[3, 1])
    np.testing.assert_allclose(osub, o[rows][:, [3, 1]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lsub, lse[[3, 1]][:, rows], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- P6: constant V
@pytest.mark.parametrize("sparse", [STREAM, BLOCK])
def test_constant_v(sparse):
    n, D = 90, 8
    q, k = _rand(15, (n, 4, D), 3.0), _rand(16, (n, 2, D), 3.0)
    c = _rand(17, (D,))
    v = np.broadcast_to(c, (n, 2, D)).copy()
    o, _ = oracle.attention(q, k, v, None, [[1, 0]], sparse)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-13)


# --------------------------------------------------------------------------- P7 / P12: router
def test_router_properties():
    n, d, dr, H = 64, 32, 8, 4
    x = _rand(18, (n, d))
    w1, w2 = _rand(19, (dr, d)), _rand(20, (H, dr))
    r = oracle.route(x, [0, n], w1, w2, 0.0, exact=True)
    perm = np.random.default_rng(21).permutation(n)
    rp = oracle.route(x[perm], [0, n], w1, w2, 0.0, exact=True)
    np.testing.assert_array_equal(r["pooled"], rp["pooled"])  # exact sums are order-free
    np.testing.assert_array_equal(r["logits"], rp["logits"])
    r4 = oracle.route(4.0 * x, [0, n], w1, w2, 0.0)  # positive homogeneity (ReLU, no bias)
    np.testing.assert_allclose(r4["logits"], 4.0 * r["logits"], rtol=1e-13)
    np.testing.assert_array_equal(r4["mask"], r["mask"])
    rz = oracle.route(np.zeros((n, d)), [0, n], w1, w2, 0.0)
    np.testing.assert_array_equal(rz["logits"], 0.0)
    np.testing.assert_array_equal(rz["mask"], 0)  # ties go to sparse
    plain = oracle.route(x, [0, n], w1, w2, 0.0)  # fp64 sums agree with the exact ones
    np.testing.assert_allclose(plain["pooled"][0], r["pooled"][0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(plain["logits"], r["logits"], rtol=1e-12, atol=1e-15)
    assert 0 < r["mask"].sum() < H  # the case is not degenerate
    # the logit is the log-odds of FULL: [l > 0] == [sigmoid(l / T) > 0.5] for any temperature
    for T in (0.1, 1.0, 10.0):
        sig = 1.0 / (1.0 + np.exp(-r["logits"] / T))
        np.testing.assert_array_equal((sig > 0.5).astype(np.int32), r["mask"])


def test_router_per_sequence_and_boundary_pooling():
    lens = [10, 300, 150]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = _rand(22, (int(cu[-1]), 16))
    w1, w2 = _rand(23, (8, 16)), _rand(24, (3, 8))
    r = oracle.route(x, cu, w1, w2)
    for b in range(3):
        rb = oracle.route(x[cu[b]:cu[b + 1]], None, w1, w2)
        np.testing.assert_array_equal(r["logits"][b], rb["logits"][0])
    rbp = oracle.route(x, cu, w1, w2, pool_head=100, pool_tail=100)
    np.testing.assert_array_equal(rbp["logits"][0], r["logits"][0])   # n <= 200: every row once
    np.testing.assert_array_equal(rbp["logits"][2], r["logits"][2])
    seq1 = x[cu[1]:cu[2]]
    manual = np.concatenate([seq1[:100], seq1[-100:]]).sum(0) / 200
    np.testing.assert_allclose(rbp["pooled"][1], manual, rtol=1e-13, atol=1e-15)
    assert oracle.pooled_rows(5, 3, 3).tolist() == [0, 1, 2, 3, 4]


# --------------------------------------------------------------------------- P8: head permutation
def test_kv_head_permutation_equivariance():
    n, G, Hkv, D = 70, 3, 3, 8
    q, k, v = _rand(25, (n, G * Hkv, D)), _rand(26, (n, Hkv, D)), _rand(27, (n, Hkv, D))
    mask = np.array([[1, 0, 0]])
    o, lse = oracle.attention(q, k, v, None, mask, STREAM)
    perm = [2, 0, 1]
    qperm = np.concatenate([q[:, g * G:(g + 1) * G] for g in perm], axis=1)
    op, lp = oracle.attention(qperm, k[:, perm], v[:, perm], None, mask[:, perm], STREAM)
    for new, old in enumerate(perm):
        np.testing.assert_array_equal(op[:, new * G:(new + 1) * G], o[:, old * G:(old + 1) * G])
        np.testing.assert_array_equal(lp[new * G:(new + 1) * G], lse[old * G:(old + 1) * G])


# --------------------------------------------------------------------------- P9: count through LSE
@pytest.mark.parametrize("sparse", [STREAM, BLOCK])
def test_zero_query_lse_counts_keys(sparse):
    n = 200
    q = np.zeros((n, 2, 8))
    k, v = _rand(28, (n, 1, 8)), _rand(29, (n, 1, 8))
    for full in (1, 0):
        _, lse = oracle.attention(q, k, v, None, [[full]], sparse)
        cnt = oracle.row_key_counts(n, bool(full), sparse)
        np.testing.assert_allclose(lse[0], np.log(cnt), rtol=0, atol=1e-13)
        np.testing.assert_array_equal(np.rint(np.exp(lse[1])).astype(int), cnt)


# --------------------------------------------------------------------------- P10: planted needle
def test_planted_needle():
    n, D = 400, 16
    sp = {"kind": "streaming", "sink": 8, "window": 32}
    q, k, v = _rand(30, (n, 1, D), 0.5), _rand(31, (n, 1, D), 0.5), _rand(32, (n, 1, D), 0.5)
    i, jstar = 350, 100                      # jstar is neither a sink nor in row i's window
    scale = D ** -0.5
    k2, v2 = k.copy(), v.copy()
    qi = q[i, 0]
    k2[jstar, 0] = (20.0 / (scale * np.linalg.norm(qi))) * qi / np.linalg.norm(qi)
    v2[jstar, 0] = 10.0
    of, _ = oracle.attention(q, k2, v2, None, [[1]], sp, rows=[i])
    assert np.all(np.abs(of[0, 0] - 10.0) < 1e-3)     # a full head retrieves the needle
    os_, _ = oracle.attention(q, k2, v2, None, [[0]], sp, rows=[i])
    o0, _ = oracle.attention(q, k, v, None, [[0]], sp, rows=[i])
    np.testing.assert_array_equal(os_, o0)           # a streaming head never sees it


# --------------------------------------------------------------------------- counters
def test_sparsity_ratios():
    m = np.array([[1, 0, 0, 0], [1, 1, 0, 1]])
    assert oracle.model_sparsity_ratio(m) == 4 / 8
    assert oracle.model_sparsity_ratio(m, [100, 300], token_weighted=True) == (3 * 100 + 1 * 300) / (400 * 4)
    sp = {"kind": "streaming", "sink": 2, "window": 3}
    esr = oracle.effective_sparsity([10], [[0]], sp, 1, 1)
    assert esr == 1 - (15 + 5 * 5) / 55  # rows 0..4 see i+1 keys, rows 5..9 see 5
    assert oracle.effective_flops(10, 128) == 5120


# --------------------------------------------------------------------------- input generator
def test_generator_is_deterministic_and_rounds_to_nearest_even():
    a = syn.draw_f32(0, 1, (3, 5), 0.5)
    b = syn.draw_f32(0, 1, (15,), 0.5)
    np.testing.assert_array_equal(a.reshape(-1), b)
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e-3], dtype=np.float32)
    bits = syn.round_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    big = syn.draw_f32(5, 2, (1 << 23) + 7)
    assert big.shape == ((1 << 23) + 7,)
    np.testing.assert_array_equal(big[:1 << 22], syn.draw_f32(5, 2, (1 << 22,)))
    np.testing.assert_array_equal(syn.round_bf16_bits(big[:4096]),
                                  torch.from_numpy(big[:4096]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))

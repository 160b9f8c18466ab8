"""Pins of the oracle's static retrieval-score head assignment ("Elastic Attention", arXiv
2601.17367; paperlayer summary, appendix C.1 "Retrieval Score Calculation" and "Sparsity
Assignment").

The score is tied to closed forms (a zero query spreads its weight evenly; a needle covering
all keys holds all of it), to brute force with Python loops, to the whole-sequence oracle
attention (its log-sum-exp of the last row, a separate code path), and to sequence
independence.  The assignment is tied to the k formula, to an independent selection by
repeated arg-max, and to nesting across sparsity ratios."""
import math

import numpy as np
import pytest

from oracle import elastic_oracle as O


def _qk(n, hq=4, hkv=2, d=8, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, hq, d)) * scale, rng.standard_normal((n, hkv, d)) * scale


@pytest.mark.parametrize("n,needle", [(10, (2, 5)), (37, (0, 1)), (64, (60, 64)), (5, (3, 100))])
def test_zero_query_spreads_evenly(n, needle):
    q, k = _qk(n)
    q[-1] = 0.0
    sq, skv = O.retrieval_scores(q, k, None, [needle])
    a, e = max(0, needle[0]), min(n, needle[1])
    assert np.allclose(sq, (e - a) / n, rtol=0, atol=1e-15)
    assert np.allclose(skv, (e - a) / n, rtol=0, atol=1e-15)


def test_whole_and_empty_needles_and_partition():
    n = 50
    q, k = _qk(n, seed=1)
    whole, _ = O.retrieval_scores(q, k, None, [(0, n)])
    empty, _ = O.retrieval_scores(q, k, None, [(7, 7)])
    left, _ = O.retrieval_scores(q, k, None, [(0, 23)])
    right, _ = O.retrieval_scores(q, k, None, [(23, n)])
    assert np.allclose(whole, 1.0, atol=1e-15) and np.all(empty == 0)
    assert np.allclose(left + right, 1.0, atol=1e-14)


def test_brute_force_loops():
    n, hq, hkv, d = 9, 4, 2, 3
    q, k = _qk(n, hq, hkv, d, seed=2)
    needle = (3, 6)
    sq, skv = O.retrieval_scores(q, k, None, [needle])
    for h in range(hq):
        g = h // (hq // hkv)
        s = [sum(q[-1, h, t] * k[j, g, t] for t in range(d)) / math.sqrt(d) for j in range(n)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        assert abs(sq[0, h] - sum(w[3:6]) / sum(w)) < 1e-14
    assert np.allclose(skv[0], [(sq[0, 0] + sq[0, 1]) / 2, (sq[0, 2] + sq[0, 3]) / 2], atol=1e-15)


def test_matches_attention_lse_of_the_last_row():
    """S = sum over the needle of exp(s_j - lse_last), lse_last from the full-head oracle."""
    n = 40
    q, k = _qk(n, seed=3, scale=2.0)
    v = np.zeros((n, 2, 8))
    _, lse = O.attention(q, k, v, None, None, None)
    needle = (11, 19)
    sq, _ = O.retrieval_scores(q, k, None, [needle])
    for h in range(4):
        s = (k[:, h // 2, :] @ q[-1, h, :]) / math.sqrt(8)
        ref = np.exp(s[11:19] - lse[h, n - 1]).sum()
        assert abs(sq[0, h] - ref) < 1e-13


def test_dominant_key_takes_the_mass():
    n, d = 30, 8
    q = np.zeros((n, 2, d))
    k = np.zeros((n, 1, d))
    k[17, 0, 0] = 1.0
    q[-1, :, 0] = 400.0                      # s_17 = 400 / sqrt(8), every other s_j = 0
    sq, _ = O.retrieval_scores(q, k, None, [(15, 20)])
    e = math.exp(-400 / math.sqrt(d))
    assert np.allclose(sq, (1 + 4 * e) / (1 + 29 * e), rtol=0, atol=1e-15)


def test_sequences_are_independent_and_empty_scores_zero():
    lens = [12, 0, 21, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k = _qk(int(cu[-1]), seed=4)
    needles = [(2, 4), (0, 5), (20, 30), (0, 1)]
    sq, skv = O.retrieval_scores(q, k, cu, needles)
    for b, (lo, hi) in enumerate(zip(cu[:-1], cu[1:])):
        if hi == lo:
            assert np.all(sq[b] == 0) and np.all(skv[b] == 0)
            continue
        one, one_kv = O.retrieval_scores(q[lo:hi], k[lo:hi], None, [needles[b]])
        assert np.array_equal(one[0], sq[b]) and np.array_equal(one_kv[0], skv[b])
    assert np.allclose(sq[3], 1.0)           # one token: it is the needle


@pytest.mark.parametrize("n,omega,k", [(8, 0.375, 5), (8, 0.0, 8), (8, 1.0, 0), (10, 0.3, 7),
                                       (10, 0.7, 3), (256, 0.5, 128), (7, 0.5, 3), (1, 0.99, 0)])
def test_assignment_count(n, omega, k):
    rng = np.random.default_rng(n)
    m = O.static_assignment(rng.random(n), omega)
    assert int(m.sum()) == k


def _select_by_argmax(scores, k):
    """Independent selection: take the best remaining unit k times (ties: lower index;
    NaN below every number)."""
    s = list(scores)
    left = set(range(len(s)))
    out = np.zeros(len(s), dtype=np.int32)
    for _ in range(k):
        best = None
        for i in sorted(left):
            if best is None:
                best = i
                continue
            a, b = s[i], s[best]
            if math.isnan(b) and not math.isnan(a):
                best = i
            elif not math.isnan(a) and not math.isnan(b) and a > b:
                best = i
        out[best] = 1
        left.remove(best)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_assignment_matches_argmax_selection(seed):
    rng = np.random.default_rng(seed)
    n = 32
    s = np.round(rng.random(n), 1)           # many ties
    s[rng.random(n) < 0.1] = np.nan
    for omega in (0.0, 0.25, 0.5, 0.6, 0.9):
        k = int(math.floor((1 - omega) * n))
        assert np.array_equal(O.static_assignment(s, omega), _select_by_argmax(s, k))


def test_assignment_nests_and_keeps_shape():
    rng = np.random.default_rng(9)
    s = rng.random((4, 8))                   # layers x KV heads
    prev = np.ones((4, 8), dtype=np.int32)
    for omega in np.linspace(0, 1, 11):
        m = O.static_assignment(s, omega)
        assert m.shape == (4, 8)
        assert np.all(m <= prev)             # a higher ratio never turns a sparse head full
        prev = m

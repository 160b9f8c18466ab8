"""Pins of the oracle's explicit per-head block lists (the consumer half of content-based
block selection; "Elastic Attention", arXiv 2601.17367, paperlayer summary section 4 and
appendix G.2 name XAttention's block selection, whose estimator is not given).

A block list that spells out a fixed block pattern must reproduce that pattern (which the
oracle evaluates by its formula, a separate code path), lists may differ per sequence and per
KV head, key blocks after the query block are ignored, and a query block with an empty list
leaves its rows without keys (o = 0, lse = -inf).  Brute force with Python loops pins a tiny
case."""
import math

import numpy as np
import pytest

from oracle import elastic_oracle as O

BLOCK = {"kind": "block", "block": 16, "sink_blocks": 1, "local_blocks": 2, "stride_blocks": 3}


def _qkv(n, hq=4, hkv=2, d=8, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, hq, d)), rng.standard_normal((n, hkv, d)),
            rng.standard_normal((n, hkv, d)))


def _csr(rows):
    """rows: list (in CSR row order) of key-block index lists."""
    rp, ci = [0], []
    for r in rows:
        ci.extend(r)
        rp.append(len(ci))
    return rp, ci


@pytest.mark.parametrize("n", [100, 160, 257])
def test_lists_spelling_out_a_pattern_reproduce_it(n):
    q, k, v = _qkv(n)
    lists = O.block_list_from_pattern(BLOCK, 1, 2, n)
    o1, l1 = O.attention(q, k, v, None, [[0, 0]], BLOCK)
    o2, l2 = O.attention(q, k, v, None, [[0, 0]], lists)
    assert np.allclose(o1, o2, rtol=0, atol=1e-13) and np.allclose(l1, l2, rtol=0, atol=1e-13)
    assert O.entries([n], [[0, 0]], lists, 4, 2) == O.entries([n], [[0, 0]], BLOCK, 4, 2)


def test_per_head_lists_later_blocks_and_empty_rows():
    n, B = 64, 16
    nqb = n // B
    q, k, v = _qkv(n, hq=2, hkv=2, seed=1)
    head0 = [[0], [0, 1], [1, 3], [0, 2, 3]]     # block 2 lists a later block (3): ignored
    head1 = [[0], [], [0, 1, 2], [3]]            # query block 1 sees nothing
    rp, ci = _csr(head0 + head1)
    lists = {"kind": "block_list", "block": B, "qblocks": nqb, "row_ptr": rp, "col_idx": ci}
    o, lse = O.attention(q, k, v, None, [[0, 0]], lists)
    # head 1, rows of query block 1: no keys
    assert np.all(o[16:32, 1] == 0) and np.all(np.isneginf(lse[1, 16:32]))
    # head 0 rows of block 2 see exactly key block 1 (the later block 3 is dropped)
    sp = O.block_list_resolve(lists, 0, 0, 2)
    assert sp["visible"][2].tolist() == [False, True, False, False]
    # the same rows through the single-head whole-sequence path with an equivalent pattern:
    # keys 16..31 only
    ref_o, ref_l = O.attention_kv(q[32:48, :1], k[16:32, :1], v[16:32, :1], None, None, None,
                                  None, q_pos=[32], k_pos=16)
    assert np.allclose(o[32:48, :1], ref_o, atol=1e-13) and np.allclose(lse[:1, 32:48], ref_l, atol=1e-13)


def test_lists_differ_per_sequence():
    lens = [48, 64]
    cu = np.concatenate([[0], np.cumsum(lens)])
    B, nqb, hkv = 16, 4, 1
    q, k, v = _qkv(sum(lens), hq=1, hkv=1, seed=2)
    seq0 = [[0], [1], [2], [0, 3]]
    seq1 = [[0], [0], [0, 1], [2, 3]]
    rp, ci = _csr(seq0 + seq1)
    lists = {"kind": "block_list", "block": B, "qblocks": nqb, "row_ptr": rp, "col_idx": ci}
    o, lse = O.attention(q, k, v, cu, [[0], [0]], lists)
    for b, rows in enumerate((seq0, seq1)):
        lo = cu[b]
        for qb, kbs in enumerate(rows):
            for t in range(qb * B, min(lens[b], qb * B + B)):
                keys = [j for kb in kbs if kb <= qb for j in range(kb * B, kb * B + B) if j <= t]
                s = [float(q[lo + t, 0] @ k[lo + j, 0]) / math.sqrt(8) for j in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                ref = sum(wi * v[lo + j, 0] for wi, j in zip(w, keys)) / sum(w)
                assert np.allclose(o[lo + t, 0], ref, atol=1e-12)
                assert abs(lse[0, lo + t] - (m + math.log(sum(w)))) < 1e-12


def test_block_lists_with_key_ranges():
    """Key-range attention honours the lists on absolute positions."""
    n, B = 96, 16
    q, k, v = _qkv(n, hq=2, hkv=1, seed=3)
    rows = [[0], [0, 1], [1, 2], [0, 3], [2, 4], [0, 4, 5]]
    rp, ci = _csr(rows)
    lists = {"kind": "block_list", "block": B, "qblocks": 6, "row_ptr": rp, "col_idx": ci}
    o, lse = O.attention(q, k, v, None, [[0]], lists)
    oa, la = O.attention_kv(q, k[:32], v[:32], None, None, [[0]], lists, q_pos=[0], k_pos=0)
    ob, lb = O.attention_kv(q, k[32:], v[32:], None, None, [[0]], lists, q_pos=[0], k_pos=32)
    om, lm = O.lse_merge(oa, la, ob, lb)
    assert np.allclose(om, o, atol=1e-12) and np.allclose(lm, lse, atol=1e-12)

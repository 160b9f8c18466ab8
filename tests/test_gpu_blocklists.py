"""GPU parity of explicit per-head block lists (CSR of key blocks per query block) against the
fp64 oracle, through the C ABI.

Small cases compare every element with seeded random lists (empty lists, missing diagonal
blocks, listed blocks after the query block, lists that differ per sequence and head), with
GQA ratios whose work items straddle several query blocks, both dtypes, and a key-range
split merged by LSE.  At 32K, lists that spell out the fixed block pattern reproduce the
fixed-pattern launch bit for bit, and seeded selection-style lists (sink block, diagonal,
random earlier blocks) match the oracle on sampled rows."""
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


random_lists, dev_lists = H.random_lists, H.dev_lists


def _draw(seed, T, hq, hkv, D, dtype="bf16", scale=0.5):
    draw = syn.draw_bf16_bits if dtype == "bf16" else syn.draw_f32
    return {"q": draw(seed, 0, (T, hq, D), scale), "k": draw(seed, 1, (T, hkv, D), scale),
            "v": draw(seed, 2, (T, hkv, D), scale)}


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


CASES = [
    # name, seqlens, hq, hkv, D, block, dtype, mask
    ("g4-d128-b64", [517], 8, 2, 128, 64, "bf16", [[0, 0]]),
    ("g7-d128-b64", [450], 14, 2, 128, 64, "bf16", [[0, 1]]),   # items straddle query blocks
    ("g1-d64-b64", [600], 2, 2, 64, 64, "bf16", [[0, 0]]),      # items span four query blocks
    ("g4-d128-b128", [700], 4, 1, 128, 128, "bf16", [[0]]),
    ("varlen", [130, 1, 300, 64], 8, 2, 128, 64, "bf16", [[0, 1], [0, 0], [1, 0], [0, 0]]),
    ("fp32-d64", [333], 8, 2, 64, 64, "f32", [[0, 0]]),
    ("g32-d128-b64", [300], 64, 2, 128, 64, "bf16", [[0, 0]]),   # items of 8 query tokens
    ("g256-d64-b128", [200], 256, 1, 64, 128, "bf16", [[0]]),    # items of one query token
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_lists_every_element(case):
    name, lens, hq, hkv, D, B, dtype, mask = case
    print(f"[case] block lists {name}", flush=True)
    T = sum(lens)
    nqb = -(-max(lens) // B)
    lists = random_lists(41 + len(name), len(lens), hkv, nqb, B)
    data = _draw(42, T, hq, hkv, D, dtype, 1.0 if dtype == "f32" else 0.5)
    q, k, v = H.to_dev(data["q"]), H.to_dev(data["k"]), H.to_dev(data["v"])
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=H.DEV)
    m = torch.tensor(mask, dtype=torch.int32, device=H.DEV)
    lse = torch.full((hq, T), float("nan"), dtype=torch.float32, device=H.DEV)
    o = ext.attn_prefill(q, k, v, cu_seqlens=cu, max_seqlen=max(lens), head_mask=m,
                         sparse=dev_lists(lists), lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], np.concatenate([[0], np.cumsum(lens)]),
                              mask, lists)
    _check(o, lse, ro, rl, name, dtype)


def test_block_lists_key_split_and_merge():
    n, hq, hkv, D, B = 400, 8, 2, 128, 64
    lists = random_lists(50, 1, hkv, -(-n // B), B)
    data = _draw(51, n, hq, hkv, D)
    q, k, v = H.to_dev(data["q"]), H.to_dev(data["k"]), H.to_dev(data["v"])
    m = torch.zeros((1, hkv), dtype=torch.int32, device=H.DEV)
    dl = dev_lists(lists)
    cut = 192
    la = torch.empty((hq, n), dtype=torch.float32, device=H.DEV)
    lb = torch.empty_like(la)
    oa = ext.attn_prefill_kv(q, k[:cut], v[:cut], q_pos=0, k_pos=0, head_mask=m, sparse=dl, lse=la)
    ob = ext.attn_prefill_kv(q, k[cut:], v[cut:], q_pos=0, k_pos=cut, head_mask=m, sparse=dl, lse=lb)
    om, lm = ext.lse_merge(oa, la, ob, lb)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], None, [[0, 0]], lists)
    _check(om, lm, ro, rl, "block lists split + merge", "bf16")


@pytest.fixture(scope="module")
def layer32k():
    w = syn.WORKLOADS["llama8b-32k-block-router"]
    data, q, k, v = H.qkv_dev(w)
    return w, data, q, k, v


def test_lists_spelling_the_pattern_match_it_bitwise_32k(layer32k):
    w, data, q, k, v = layer32k
    n, hq, hkv = q.shape[0], q.shape[1], k.shape[1]
    mask = torch.tensor([[1, 0, 0, 1, 0, 1, 0, 0]], dtype=torch.int32, device=H.DEV)
    lists = oracle.block_list_from_pattern(w.sparse, 1, hkv, n)
    l1 = torch.empty((hq, n), dtype=torch.float32, device=H.DEV)
    l2 = torch.empty_like(l1)
    o1 = ext.attn_prefill(q, k, v, max_seqlen=n, head_mask=mask, sparse=w.sparse, lse=l1)
    o2 = ext.attn_prefill(q, k, v, max_seqlen=n, head_mask=mask, sparse=dev_lists(lists), lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    ent = ext.attn_entries([n], mask.cpu().numpy().tolist(), hq, hkv, lists)
    assert ent == ext.attn_entries([n], mask.cpu().numpy().tolist(), hq, hkv, w.sparse)


def test_selection_style_lists_32k(layer32k):
    """Per head: the sink block, the diagonal and about 8% of the earlier blocks, seeded."""
    w, data, q, k, v = layer32k
    n, hq, hkv, B = q.shape[0], q.shape[1], k.shape[1], 128
    nqb = n // B
    rng = np.random.default_rng(60)
    rp, ci = [0], []
    for g in range(hkv):
        for qb in range(nqb):
            kbs = {0, qb} | set(np.nonzero(rng.random(qb) < 0.08)[0].tolist())
            ci.extend(sorted(kbs))
            rp.append(len(ci))
    lists = {"kind": "block_list", "block": B, "qblocks": nqb, "row_ptr": rp, "col_idx": ci}
    zeros = [[0] * hkv]
    lse = torch.empty((hq, n), dtype=torch.float32, device=H.DEV)
    o = ext.attn_prefill(q, k, v, max_seqlen=n, head_mask=torch.tensor(zeros, dtype=torch.int32, device=H.DEV),
                         sparse=dev_lists(lists), lse=lse)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([syn.spread_rows(n, 40, 61), [127, 128, 16383, 16384]]))
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], None, zeros, lists, rows=rows, workers=16)
    H.assert_bf16_close(H.to_f64(o[torch.from_numpy(rows).to(H.DEV)]), ro, "32K selection lists")
    np.testing.assert_allclose(H.to_f64(lse)[:, rows], rl, rtol=0, atol=H.BF16_LSE_ATOL)

"""GPU parity of the static retrieval-score head assignment ("Elastic Attention", arXiv
2601.17367; paperlayer summary, appendix C.1) against the fp64 oracle, through the C ABI.

Scores: every (sequence, head) on seeded inputs -- varlen batches with an empty sequence,
needles inside, across chunk edges, clipped and empty, GQA ratios that need one and several
head slices, both head sizes and dtypes, lengths spanning several key chunks with a ragged
tail -- and on the 32K layer's q/k.  Inputs are exact bf16/fp32 values on both sides, so the
only GPU error is fp32 accumulation: scores within 1e-4 absolute.  Assignment: the mask is
bit-exact against the oracle on the same fp32 scores (ties and NaN included), and a chain
scores -> assignment -> attention with that forced mask matches the oracle."""
import math

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


CASES = [
    # name, seqlens, hq, hkv, D, dtype, needles, scale
    ("g4-d128", [2500], 32, 8, 128, "bf16", [(1000, 1100)], 0.5),
    ("g7-d128-varlen", [700, 0, 1500, 1], 28, 4, 128, "bf16", [(3, 9), (0, 4), (1020, 1030), (0, 1)], 0.5),
    ("g12-d64", [1300], 12, 1, 64, "bf16", [(0, 1300)], 0.5),
    ("g1-d64-clip", [900], 4, 4, 64, "bf16", [(880, 5000)], 0.5),
    ("g16-empty-needle", [333, 1025], 32, 2, 128, "bf16", [(5, 5), (-10, 3)], 0.5),
    ("fp32-d128", [1500], 8, 2, 128, "f32", [(100, 400)], 1.0),
    ("fp32-d64-varlen", [64, 1100], 16, 4, 64, "f32", [(60, 64), (1023, 1025)], 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_scores_every_head(case):
    name, lens, hq, hkv, D, dtype, needles, scale = case
    print(f"[case] retrieval scores {name}", flush=True)
    T = sum(lens)
    draw = syn.draw_bf16_bits if dtype == "bf16" else syn.draw_f32
    q = draw(70, 0, (T, hq, D), scale)
    k = draw(70, 1, (T, hkv, D), scale)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    nd = torch.tensor(needles, dtype=torch.int32, device=H.DEV)
    sq, skv = ext.retrieval_scores(H.to_dev(q), H.to_dev(k), nd,
                                   cu_seqlens=torch.from_numpy(cu).to(H.DEV), max_seqlen=max(lens))
    torch.cuda.synchronize()
    rq, rkv = oracle.retrieval_scores(q, k, cu, needles)
    np.testing.assert_allclose(H.to_f64(sq), rq, rtol=0, atol=2e-5)
    np.testing.assert_allclose(H.to_f64(skv), rkv, rtol=0, atol=2e-5)


def test_scores_32k_layer():
    w = syn.WORKLOADS["llama8b-32k-block-router"]
    data = syn.make_qkv(w)
    n = w.seqlens[0]
    for needle in ((16000, 16064), (0, 128), (n - 64, n)):
        nd = torch.tensor([needle], dtype=torch.int32, device=H.DEV)
        sq, skv = ext.retrieval_scores(H.to_dev(data["q"]), H.to_dev(data["k"]), nd)
        torch.cuda.synchronize()
        rq, rkv = oracle.retrieval_scores(data["q"], data["k"], None, [needle])
        print(f"[parity] 32K needle {needle}: max |d| {np.abs(H.to_f64(sq) - rq).max():.2e}", flush=True)
        np.testing.assert_allclose(H.to_f64(sq), rq, rtol=0, atol=1e-4)
        np.testing.assert_allclose(H.to_f64(skv), rkv, rtol=0, atol=1e-4)


@pytest.mark.parametrize("shape,seed", [((32, 8), 0), ((1, 1), 1), ((4, 7), 2), ((128, 32), 3),
                                        ((128, 128), 4)])
def test_assignment_bit_exact(shape, seed):
    rng = np.random.default_rng(seed)
    s = np.round(rng.random(shape), 2).astype(np.float32)   # many ties
    s[rng.random(shape) < 0.05] = np.nan
    dev = torch.from_numpy(s).to(H.DEV)
    for omega in (0.0, 0.3, 0.375, 0.5, 0.7, 0.99, 1.0):
        m = ext.static_assignment(dev, omega)
        torch.cuda.synchronize()
        ref = oracle.static_assignment(s.astype(np.float64), omega)
        assert np.array_equal(m.cpu().numpy(), ref), (shape, omega)
        assert int(m.sum()) == int(math.floor((1 - omega) * s.size))


def test_scores_assignment_attention_chain():
    """Scores of two 'layers' (different seeds), one assignment over both, and each layer's
    slice as the forced mask of the attention call."""
    n, hq, hkv, D = 777, 16, 4, 128
    sparse = {"kind": "streaming", "sink": 4, "window": 64}
    layers = []
    for seed in (80, 81):
        q = syn.draw_bf16_bits(seed, 0, (n, hq, D), 0.5)
        k = syn.draw_bf16_bits(seed, 1, (n, hkv, D), 0.5)
        v = syn.draw_bf16_bits(seed, 2, (n, hkv, D), 0.5)
        layers.append((q, k, v))
    nd = torch.tensor([[300, 340]], dtype=torch.int32, device=H.DEV)
    sc = torch.cat([ext.retrieval_scores(H.to_dev(q), H.to_dev(k), nd)[1] for q, k, _ in layers])
    mask = ext.static_assignment(sc, 0.5)                       # [2 layers, 4 KV heads]
    torch.cuda.synchronize()
    ref_mask = oracle.static_assignment(H.to_f64(sc), 0.5)
    assert np.array_equal(mask.cpu().numpy(), ref_mask) and int(mask.sum()) == 4
    for li, (q, k, v) in enumerate(layers):
        o = ext.attn_prefill(H.to_dev(q), H.to_dev(k), H.to_dev(v), max_seqlen=n,
                             head_mask=mask[li:li + 1].contiguous(), sparse=sparse)
        torch.cuda.synchronize()
        ro, _ = oracle.attention(q, k, v, None, ref_mask[li:li + 1], sparse)
        H.assert_bf16_close(H.to_f64(o), ro, f"chain layer {li}")

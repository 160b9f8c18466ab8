"""Packed batches of many short sequences through the C ABI, against the fp64 oracle.

More than 64 sequences take the router's wave-wide slab search (below that a workgroup walks
the sequences one by one); more than 1,024 sequences, or more than 16,384 (sequence, KV head)
mask entries, take the scheduler past its LDS caches of sequence offsets and the head mask.
Every logit and every attention output element is compared; empty sequences are mixed in.

Method: "Elastic Attention" (arXiv 2601.17367), paperlayer summary section 3 "Attention
Router" (one pooled decision per sequence and KV head), section 3 "Efficient Deployment" and
appendix D.1 "Sparse Inference" (one unified launch over a packed batch of mixed heads)."""
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


def _lens(seed: int, batch: int, longest: int) -> list:
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, longest + 1, size=batch)
    lens[rng.random(batch) < 0.1] = 0          # about one sequence in ten is empty
    return [int(x) for x in lens]


@pytest.mark.parametrize("batch", [100, 1500])
def test_router_many_sequences(batch):
    lens = _lens(40 + batch, batch, 40)
    T, d, hkv = sum(lens), 256, 6
    hidden = syn.draw_bf16_bits(41, 3, (T, d))
    w1 = syn.draw_f32(41, 4, (64, d), 0.1)
    w2 = syn.draw_f32(41, 5, (hkv, 64), 0.1)
    cu_np = np.cumsum([0] + lens).astype(np.int32)
    cu = torch.tensor(cu_np, device=H.DEV)
    for ph, pt in ((0, 0), (3, 2)):
        print(f"[many] router batch {batch} T {T} pool {ph}/{pt}", flush=True)
        logits, mask = ext.route(H.to_dev(hidden), H.to_dev(w1), H.to_dev(w2), cu_seqlens=cu,
                                 pool_head=ph, pool_tail=pt)
        ref = oracle.route(hidden, cu_np, w1, w2, 0.0, pool_head=ph, pool_tail=pt)
        lg = logits.cpu().numpy()
        np.testing.assert_allclose(lg, ref["logits"], rtol=1e-4, atol=1e-6)
        outside = np.abs(ref["logits"]) >= 1e-5
        np.testing.assert_array_equal(mask.cpu().numpy()[outside], ref["mask"][outside])
        empty = np.array(lens) == 0
        assert np.all(lg[empty] == 0) and np.all(mask.cpu().numpy()[empty] == 0)


CASES = [
    # batch > 1024: sequence offsets read from the workspace, not the LDS cache
    ("1500 seqs, G 2, streaming", 1500, 40, 4, 2, {"kind": "streaming", "sink": 3, "window": 9}),
    # 1400 x 12 = 16,800 mask entries > 16,384: the head mask read from global memory
    ("1400 seqs, 12 KV heads, block", 1400, 30, 12, 12,
     {"kind": "block", "block": 64, "sink_blocks": 1, "local_blocks": 0, "stride_blocks": 0}),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_many_sequences(case):
    name, batch, longest, hq, hkv, sparse = case
    lens = _lens(batch + hq, batch, longest)
    T, D = sum(lens), 64
    seed = 1000 + batch
    data = {"q": syn.draw_bf16_bits(seed, 0, (T, hq, D), 0.5),
            "k": syn.draw_bf16_bits(seed, 1, (T, hkv, D), 0.5),
            "v": syn.draw_bf16_bits(seed, 2, (T, hkv, D), 0.5)}
    mask = np.random.default_rng(seed).integers(0, 2, size=(batch, hkv)).astype(np.int32)
    cu = np.cumsum([0] + lens).astype(np.int32)
    print(f"[many] attention {name}: T {T}", flush=True)
    lse = torch.full((hq, T), float("nan"), dtype=torch.float32, device=H.DEV)
    o = ext.attn_prefill(H.to_dev(data["q"]), H.to_dev(data["k"]), H.to_dev(data["v"]),
                         cu_seqlens=torch.tensor(cu, device=H.DEV), max_seqlen=max(lens),
                         head_mask=torch.tensor(mask, device=H.DEV), sparse=sparse, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], cu, mask, sparse, workers=8)
    got, gl = H.to_f64(o), H.to_f64(lse)
    H.assert_bf16_close(got, ro, name)
    np.testing.assert_allclose(gl, rl, rtol=0, atol=H.BF16_LSE_ATOL, err_msg=name)

"""One sequence long enough that q and o pass 2^31 bytes and 2^31 elements, through the C ABI,
against the fp64 oracle on sampled rows.

540,013 tokens x 32 query heads x D 128 in bf16 is 4.4 GB per tensor, so byte offsets past
2^31 start at token 262,144 and element offsets past 2^31 at token 524,288; the rows sampled
sit on both sides of each boundary and at the ragged end.  Two KV heads are full (causal over
the whole sequence) and six stream (sink 128, window 1024); the oracle is run on KV heads 0
(full), 1 (streaming) and 7 (full) with their four query heads each, every element of the
sampled rows compared.

Method: "Elastic Attention" (arXiv 2601.17367), paperlayer summary section 2 "Hybrid Head
Mechanism" (full and sparse heads in one layer), section 4 "Length Extrapolation Capability
Testing" (long contexts), appendix D.1 "Sparse Inference" (sink + window streaming)."""
import numpy as np
import pytest
import torch

import oracle
from synth import inputs as syn
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

T, HQ, HKV, D = 540_013, 32, 8, 128
G = HQ // HKV
MASK = [[1, 0, 0, 0, 0, 0, 0, 1]]
SPARSE = {"kind": "streaming", "sink": 128, "window": 1024}
ROWS = [0, 1, 127, 128, 1151, 1152, 262_143, 262_144, 262_145, 524_287, 524_288, 524_289,
        T - 64, T - 2, T - 1]
KV_CHECK = [0, 1, 7]


def test_attention_past_2gib_offsets():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import hybrid_sparse_full_elastic_amd as ext  # no fallback: must load the HIP library
    print(f"[large] T {T}: drawing inputs", flush=True)
    q = syn.draw_bf16_bits(91, syn.TAG_Q, (T, HQ, D), 0.5)
    k = syn.draw_bf16_bits(91, syn.TAG_K, (T, HKV, D), 0.5)
    v = syn.draw_bf16_bits(91, syn.TAG_V, (T, HKV, D), 0.5)
    assert q.nbytes > (1 << 31) and q.size > (1 << 31)
    lse = torch.full((HQ, T), float("nan"), dtype=torch.float32, device=H.DEV)
    print("[large] attention", flush=True)
    o = ext.attn_prefill(H.to_dev(q), H.to_dev(k), H.to_dev(v), max_seqlen=T,
                         head_mask=torch.tensor(MASK, dtype=torch.int32, device=H.DEV),
                         sparse=SPARSE, lse=lse)
    torch.cuda.synchronize()
    rows = torch.tensor(ROWS, device=H.DEV)
    got = H.to_f64(o.index_select(0, rows))
    got_lse = H.to_f64(lse.index_select(1, rows))
    del o, lse
    torch.cuda.empty_cache()
    qh = [g * G + j for g in KV_CHECK for j in range(G)]
    print("[large] oracle", flush=True)
    ro, rl = oracle.attention(np.ascontiguousarray(q[:, qh]), np.ascontiguousarray(k[:, KV_CHECK]),
                              np.ascontiguousarray(v[:, KV_CHECK]), None,
                              [[MASK[0][g] for g in KV_CHECK]], SPARSE, rows=ROWS, workers=8)
    H.assert_bf16_close(got[:, qh], ro, "540K tokens, sampled rows")
    np.testing.assert_allclose(got_lse[qh], rl, rtol=0, atol=H.BF16_LSE_ATOL)

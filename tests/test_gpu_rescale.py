"""GPU parity on inputs whose scores climb steeply along the keys, so that the running
maximum of the online softmax has to be raised again and again within one item (tiles whose
weights outgrow the current maximum are redone with their own maximum), against the fp64
oracle through the C ABI.  Rising, falling and flat heads share one launch, with full and
streaming heads, and the LSE of every row is checked too."""
import numpy as np
import pytest
import torch

import oracle
from synth import inputs as syn
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _bf16(x):
    return syn.round_bf16_bits(np.ascontiguousarray(x, dtype=np.float32))


@pytest.mark.parametrize("slope", [0.05, 0.4, 2.0])
def test_steep_scores(slope):
    print(f"[case] rising scores slope {slope}", flush=True)
    import hybrid_sparse_full_elastic_amd as ext
    n, hq, hkv, D = 1000, 8, 2, 128
    rng = np.random.default_rng(90)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    j = np.arange(n, dtype=np.float64)
    q = rng.standard_normal((n, hq, D)) * 0.3
    k = rng.standard_normal((n, hkv, D)) * 0.3
    v = rng.standard_normal((n, hkv, D))
    q[:, :, :] += 4.0 * u                          # every query points along u
    k[:, 0, :] += (slope * j)[:, None] * u         # KV head 0: scores rise with j
    k[:, 1, :] -= (slope * j)[:, None] * u         # KV head 1: scores fall with j
    q, k, v = _bf16(q), _bf16(k), _bf16(v)
    for mask, sparse in (([[1, 1]], None), ([[1, 0]], {"kind": "streaming", "sink": 16, "window": 200})):
        lse = torch.empty((hq, n), dtype=torch.float32, device=H.DEV)
        m = torch.tensor(mask, dtype=torch.int32, device=H.DEV)
        o = ext.attn_prefill(H.to_dev(q), H.to_dev(k), H.to_dev(v), max_seqlen=n, head_mask=m,
                             sparse=sparse or {"kind": "streaming", "sink": 0, "window": 1}, lse=lse)
        torch.cuda.synchronize()
        ro, rl = oracle.attention(q, k, v, None, mask, sparse or {"kind": "streaming", "sink": 0, "window": 1})
        H.assert_bf16_close(H.to_f64(o), ro, f"slope {slope} mask {mask}")
        got = H.to_f64(lse)
        print(f"[parity] lse max |d| {np.abs(got - rl).max():.2e}, max lse {rl.max():.1f}", flush=True)
        # scores here reach ~550 (natural units); a fp32 sum of D = 128 exact bf16 products
        # carries a relative error up to ~D * 2^-24 = 7.6e-6 of the score, which the lse
        # inherits from the row maximum
        np.testing.assert_allclose(got, rl, rtol=1e-5, atol=H.BF16_LSE_ATOL)

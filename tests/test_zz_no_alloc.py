"""The allocation-free attention entry point (elastic_attn_prefill_noalloc, for callers that
cannot allocate device memory) against the workspace entry point it varies, through the C ABI.

Both run the same scheduler and attention kernels; the variant keeps the scheduler's work list
in the library's per-GPU scratch array instead of a caller workspace, so its outputs must be
bit-identical.  Two calls in a row, the second smaller than the first, show that the contents
the first call leaves in the shared array never leak into the second."""
import numpy as np
import pytest
import torch

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


CALLS = [
    # seqlens, hq, hkv, D, dtype, sparse, mask
    ([3000, 1777, 0, 513], 32, 8, 128, "bf16", {"kind": "streaming", "sink": 64, "window": 300},
     [[1, 0, 1, 0, 0, 1, 1, 0], [0, 0, 1, 1, 0, 1, 0, 1], [1, 1, 1, 1, 0, 0, 0, 0],
      [0, 1, 0, 1, 1, 0, 1, 0]]),
    ([700], 8, 2, 64, "bf16",
     {"kind": "block", "block": 64, "sink_blocks": 1, "local_blocks": 2, "stride_blocks": 3}, [[0, 1]]),
    ([257, 31], 12, 4, 128, "f32", {"kind": "streaming", "sink": 4, "window": 40},
     [[1, 0, 0, 1], [0, 1, 1, 0]]),
]


def _inputs(i, seqlens, hq, hkv, D, dtype):
    T = sum(seqlens)
    draw = syn.draw_bf16_bits if dtype == "bf16" else syn.draw_f32
    return [H.to_dev(draw(60 + i, t, (T, h, D), 0.5)) for t, h in ((0, hq), (1, hkv), (2, hkv))]


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_noalloc_matches_workspace_entry(order):
    calls = list(enumerate(CALLS))
    if order == "small_then_large":
        calls = calls[::-1]
    for i, (seqlens, hq, hkv, D, dtype, sparse, mask) in calls:
        print(f"[noalloc] call {i}: seqlens {seqlens} {hq}/{hkv} D {D} {dtype} {sparse['kind']}",
              flush=True)
        q, k, v = _inputs(i, seqlens, hq, hkv, D, dtype)
        T = q.shape[0]
        cu = torch.tensor(np.concatenate([[0], np.cumsum(seqlens)]), dtype=torch.int32, device=H.DEV)
        m = torch.tensor(mask, dtype=torch.int32, device=H.DEV)
        o_ref = torch.full_like(q, float("nan"))
        l_ref = torch.full((hq, T), float("nan"), dtype=torch.float32, device=H.DEV)
        ext.attn_prefill(q, k, v, cu_seqlens=cu, max_seqlen=max(seqlens), head_mask=m,
                         sparse=sparse, out=o_ref, lse=l_ref)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((hq, T), float("nan"), dtype=torch.float32, device=H.DEV)
        ext.attn_prefill_noalloc(q, k, v, o, cu_seqlens=cu, max_seqlen=max(seqlens), head_mask=m,
                                 sparse=sparse, lse=lse)
        torch.cuda.synchronize()
        assert not torch.isnan(o).any() and not torch.isnan(lse).any()
        assert torch.equal(o.view(torch.int16) if dtype == "bf16" else o.view(torch.int32),
                           o_ref.view(torch.int16) if dtype == "bf16" else o_ref.view(torch.int32))
        assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32))

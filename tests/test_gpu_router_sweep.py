"""Seeded randomized sweep of the Attention Router through the C ABI against the fp64 oracle.

Each case draws a packed batch (1 to 300 sequences, about one in ten empty), the model width
(8 to 4096, a multiple of 8: one ragged 64-column strip or many), the router width (1 to 256)
and KV-head count (1 to 64), boundary pooling or the whole sequence, the hidden dtype (bf16,
or bf16 values in fp32) and the threshold (0, or a random value).  Batches past 64 sequences
take the slab search instead of the walk over sequences; batch sizes past the few-slab limit
take the many-slab pooling shape.  Every logit is compared, and the mask wherever the logit
is clear of the threshold by more than the fp32 summation error; empty sequences give logit
0 and mask 0.  The loop stops at the first failing case and names its seed.

Method: "Elastic Attention" (arXiv 2601.17367), paperlayer summary section 3 "Attention
Router" (pooled hidden states, task MLP and router MLP, one logit per KV head, a threshold
between full and sparse attention) and appendix H.4 "Router Input Length" (boundary pooling
over the first and last tokens)."""
import numpy as np
import pytest
import torch

import oracle
from synth import inputs as syn
from tests import gpu_helpers as H

N_CASES = 40
MAX_ELEMS = 6_000_000  # hidden elements per case: the oracle's pooled mean stays fast


def draw_case(i: int) -> dict:
    """The i-th seeded case (host only)."""
    rng = np.random.default_rng([91, i])
    batch = int(rng.choice([1, 2, 5, 17, 64, 65, 130, 300]))
    d = int(rng.choice([8, 64, 200, 1000, 4096]))
    lmax = int(max(1, min(3000, MAX_ELEMS // (d * batch))))
    lens = rng.integers(0, lmax + 1, size=batch)
    lens[rng.random(batch) < 0.1] = 0
    pool = (0, 0) if rng.random() < 0.5 else (int(rng.integers(0, 201)), int(rng.integers(0, 201)))
    return {"seed": i, "lens": [int(x) for x in lens], "d": d,
            "dr": int(rng.integers(1, 257)), "hkv": int(rng.integers(1, 65)),
            "pool": pool, "dtype": "fp32" if rng.random() < 0.25 else "bf16",
            "threshold": 0.0 if rng.random() < 0.7 else float(rng.normal(0.0, 0.05))}


def run_case(ext, c: dict) -> None:
    lens, d, dr, hkv = c["lens"], c["d"], c["dr"], c["hkv"]
    T = sum(lens)
    seed = 5000 + c["seed"]
    hidden = syn.draw_bf16_bits(seed, 3, (T, d))
    if c["dtype"] == "fp32":
        hidden = (hidden.astype(np.uint32) << 16).view(np.float32)
    w1 = syn.draw_f32(seed, 4, (dr, d), 0.1)
    w2 = syn.draw_f32(seed, 5, (hkv, dr), 0.1)
    cu_np = np.cumsum([0] + lens).astype(np.int32)
    ph, pt = c["pool"]
    print(f"[router sweep] case {c['seed']}: batch {len(lens)} T {T} d {d} dr {dr} hkv {hkv} "
          f"pool {ph}/{pt} {c['dtype']} threshold {c['threshold']:.4f}", flush=True)
    logits, mask = ext.route(H.to_dev(hidden), H.to_dev(w1), H.to_dev(w2),
                             cu_seqlens=torch.tensor(cu_np, device=H.DEV), threshold=c["threshold"],
                             pool_head=ph, pool_tail=pt)
    ref = oracle.route(hidden, cu_np, w1, w2, c["threshold"], pool_head=ph, pool_tail=pt)
    lg, mk = logits.cpu().numpy(), mask.cpu().numpy()
    np.testing.assert_allclose(lg, ref["logits"], rtol=1e-4, atol=1e-6,
                               err_msg=f"router sweep case {c['seed']}")
    clear = np.abs(ref["logits"] - c["threshold"]) >= 1e-4 * np.abs(ref["logits"]) + 1e-5
    np.testing.assert_array_equal(mk[clear], ref["mask"][clear], err_msg=f"router sweep case {c['seed']}")
    empty = np.array(lens) == 0
    assert np.all(lg[empty] == 0), c["seed"]
    assert np.all(mk[empty] == (0.0 > c["threshold"])), c["seed"]


def test_host_cases_cover_the_paths():
    cases = [draw_case(i) for i in range(N_CASES)]
    assert any(len(c["lens"]) > 64 for c in cases) and any(len(c["lens"]) <= 64 for c in cases)
    assert any(c["pool"] != (0, 0) for c in cases) and any(c["pool"] == (0, 0) for c in cases)
    assert {c["dtype"] for c in cases} == {"bf16", "fp32"}
    assert any(c["threshold"] != 0.0 for c in cases)
    assert any(0 in c["lens"] for c in cases)
    assert any(c["d"] % 64 != 0 for c in cases) and any(c["d"] == 4096 for c in cases)


@pytest.mark.gpu
def test_router_sweep():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import hybrid_sparse_full_elastic_amd as ext  # no fallback: must load the HIP library
    for i in range(N_CASES):
        run_case(ext, draw_case(i))
    torch.cuda.synchronize()

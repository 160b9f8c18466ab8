"""Seeded randomized sweep of the hybrid-head attention against the fp64 oracle, through the
C ABI, every output element compared.

Each GQA ratio G in {1, 2, 3, 4, 5, 6, 7, 8, 16} runs a fixed list of seeded cases.  A case
draws its head dim (64 / 128), dtype (mostly bf16, some fp32), KV-head count, a packed batch
of one to three sequences of 0..700 tokens, a random full/sparse mask per (sequence, KV head),
and a sparse pattern: streaming with random sink and window, the block pattern with random
block size, sink, local and stride, or random per-head block lists.  Work items hold
256 / G query tokens (bf16), so G = 3, 5, 6, 7 leave padded rows in every item and G = 16
gives 16-token items; ragged sequence ends and empty sequences hit every edge of the tile
schedule.  The loop stops at the first failing case and names its seed.

Method: "Elastic Attention" (arXiv 2601.17367), paperlayer summary section 2 "Hybrid Head
Mechanism" and "Takeaways & Limitations" (GQA: a group of query heads shares one KV head),
section 3 "Attention Router" (one full/sparse decision per KV head), appendix D.1 "Sparse
Inference" (sink + window streaming, block-sparse patterns)."""
import numpy as np
import pytest
import torch

import oracle
from synth import inputs as syn
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

ext = None
CASES_PER_G = 6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    global ext
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import hybrid_sparse_full_elastic_amd as m  # no fallback: must load the HIP library
    ext = m
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def draw_case(G: int, i: int) -> dict:
    """The i-th seeded case for GQA ratio G (host only: shapes, pattern, mask)."""
    rng = np.random.default_rng([77, G, i])
    D = int(rng.choice([64, 128]))
    dtype = "f32" if i % 6 == 5 else "bf16"
    hkv = int(rng.integers(1, 3 if G >= 8 else 4))
    nseq = int(rng.integers(1, 4))
    lens = [int(x) for x in rng.integers(0, 701, size=nseq)]
    if i == 0:
        lens = [int(rng.integers(600, 701))]          # one long single sequence
    if sum(lens) == 0:
        lens[0] = 1
    nseq = len(lens)
    kind = ["streaming", "block", "block_list"][i % 3]
    if kind == "streaming":
        sparse = {"kind": "streaming", "sink": int(rng.integers(0, 100)),
                  "window": int(rng.integers(1, 400))}
    elif kind == "block":
        sparse = {"kind": "block", "block": int(rng.choice([64, 128])),
                  "sink_blocks": int(rng.integers(0, 3)), "local_blocks": int(rng.integers(0, 5)),
                  "stride_blocks": int(rng.choice([0, 2, 3, 4, 6]))}
    else:
        B = int(rng.choice([64, 128]))
        nqb = -(-max(lens) // B)
        sparse = H.random_lists(int(rng.integers(1 << 30)), nseq, hkv, max(nqb, 1), B,
                                density=float(rng.uniform(0.1, 0.6)))
    mask = rng.integers(0, 2, size=(nseq, hkv)).astype(np.int32)
    if i == 1:
        mask[:] = 0                                    # every head sparse
    return {"seed": int(rng.integers(1 << 30)), "D": D, "dtype": dtype, "hkv": hkv, "hq": G * hkv,
            "lens": lens, "sparse": sparse, "mask": mask}


def run_case(c: dict) -> None:
    T = sum(c["lens"])
    draw = syn.draw_bf16_bits if c["dtype"] == "bf16" else syn.draw_f32
    scale = 0.5 if c["dtype"] == "bf16" else 1.0
    data = {"q": draw(c["seed"], 0, (T, c["hq"], c["D"]), scale),
            "k": draw(c["seed"], 1, (T, c["hkv"], c["D"]), scale),
            "v": draw(c["seed"], 2, (T, c["hkv"], c["D"]), scale)}
    cu = np.concatenate([[0], np.cumsum(c["lens"])]).astype(np.int32)
    sp = c["sparse"]
    sp_dev = H.dev_lists(sp) if sp["kind"] == "block_list" else sp
    lse = torch.full((c["hq"], T), float("nan"), dtype=torch.float32, device=H.DEV)
    o = ext.attn_prefill(H.to_dev(data["q"]), H.to_dev(data["k"]), H.to_dev(data["v"]),
                         cu_seqlens=torch.tensor(cu, device=H.DEV), max_seqlen=max(c["lens"]),
                         head_mask=torch.tensor(c["mask"], device=H.DEV), sparse=sp_dev, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], cu, c["mask"], sp, workers=8)
    got, gl = H.to_f64(o), H.to_f64(lse)
    what = (f"G={c['hq'] // c['hkv']} D={c['D']} {c['dtype']} lens={c['lens']} hkv={c['hkv']} "
            f"mask={c['mask'].tolist()} sparse={ {k: v for k, v in sp.items() if k not in ('row_ptr', 'col_idx')} }")
    if c["dtype"] == "bf16":
        H.assert_bf16_close(got, ro, what)
        atol = H.BF16_LSE_ATOL
    else:
        H.assert_f32_close(got, ro, what)
        atol = 1e-5
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(gl), ~fin), what        # rows without keys: lse = -inf
    np.testing.assert_allclose(gl[fin], rl[fin], rtol=0, atol=atol, err_msg=what)
    assert np.all(got[np.transpose(~fin)] == 0), what          # ... and o = 0


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8, 16])
def test_seeded_shape_and_gqa_sweep(G):
    for i in range(CASES_PER_G):
        c = draw_case(G, i)
        print(f"[sweep] G={G} case {i} seed {c['seed']} lens {c['lens']} D {c['D']} {c['dtype']} "
              f"{c['sparse']['kind']}", flush=True)
        run_case(c)

"""GPU parity of libelastic against the fp64 oracle, through the C ABI.

Small cases compare every output element (several query and key tiles, ragged tails, GQA
ratios 1/4/7/8 and 32/64/128/256 (items of 8 query tokens down to one), head dims 64/128,
every sparse pattern, packed variable-length batches; the seeded sweep in test_gpu_sweep.py
adds G = 2, 3, 5, 6, 16 and random patterns).
The five workload shapes are checked at full size in the launch configuration the
benchmark times, on a deterministic row sample the oracle computes exactly: per sequence the
first 2 * (sink + window) rows, every 16th block of 128 rows and the last block, for every
query head (64K and the packed batch: the first and last query head of every KV group).  Attention parity uses
the head mask the GPU router produced (a head inside the router's tie band would otherwise
turn a correct kernel into a large error); the router is checked on its own: mask bits
must agree wherever the oracle logit is at least 1e-3 away from the threshold.
"""
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


def _bf16_case(seed, seqlens, hq, hkv, D, scale=0.5, dtype="bf16"):
    T = int(sum(seqlens))
    draw = syn.draw_bf16_bits if dtype == "bf16" else syn.draw_f32
    return {"q": draw(seed, 0, (T, hq, D), scale), "k": draw(seed, 1, (T, hkv, D), scale),
            "v": draw(seed, 2, (T, hkv, D), scale)}


def _run_attn(data, seqlens, mask, sparse, lse=True):
    q, k, v = H.to_dev(data["q"]), H.to_dev(data["k"]), H.to_dev(data["v"])
    T, hq, _ = q.shape
    cu = torch.tensor(np.concatenate([[0], np.cumsum(seqlens)]), dtype=torch.int32, device=H.DEV)
    m = None if mask is None else torch.tensor(np.asarray(mask), dtype=torch.int32, device=H.DEV)
    l = torch.full((hq, T), float("nan"), dtype=torch.float32, device=H.DEV) if lse else None
    o = ext.attn_prefill(q, k, v, cu_seqlens=cu, max_seqlen=max(seqlens), head_mask=m, sparse=sparse, lse=l)
    torch.cuda.synchronize()
    return H.to_f64(o), (H.to_f64(l) if lse else None)


SMALL = [
    # name, seqlens, hq, hkv, D, sparse, mask
    ("stream-g4-d128-ragged", [300], 8, 2, 128, {"kind": "streaming", "sink": 4, "window": 50}, [[1, 0]]),
    ("stream-g4-d64", [450], 8, 2, 64, {"kind": "streaming", "sink": 70, "window": 130}, [[0, 1]]),
    ("block64-g4-d128", [517], 8, 2, 128,
     {"kind": "block", "block": 64, "sink_blocks": 1, "local_blocks": 2, "stride_blocks": 3}, [[0, 1]]),
    ("block128-g1-d64", [700], 2, 2, 64,
     {"kind": "block", "block": 128, "sink_blocks": 1, "local_blocks": 1, "stride_blocks": 2}, [[0, 0]]),
    ("block128-g4-nostride", [640], 4, 1, 128,
     {"kind": "block", "block": 128, "sink_blocks": 0, "local_blocks": 1, "stride_blocks": 0}, [[0]]),
    ("stream-g7-d128", [333], 14, 2, 128, {"kind": "streaming", "sink": 16, "window": 100}, [[0, 1]]),
    ("full-g8-d64", [260], 8, 1, 64, None, None),
    ("varlen-mixed", [1, 129, 64, 250, 0, 77], 8, 2, 128, {"kind": "streaming", "sink": 3, "window": 40},
     [[1, 0], [0, 1], [0, 0], [1, 1], [0, 1], [0, 0]]),
    ("stream-window-covers-all", [200], 4, 1, 128, {"kind": "streaming", "sink": 0, "window": 4096}, [[0]]),
    # large GQA ratios: items of 8, 4, 2 and 1 query tokens (256 / G), a wave's 32 rows a
    # fraction of one token's heads
    ("full-g32-d128", [150], 64, 2, 128, None, None),
    ("stream-g64-d64", [137], 64, 1, 64, {"kind": "streaming", "sink": 5, "window": 40}, [[0]]),
    ("block64-g128-d128", [200], 128, 1, 128,
     {"kind": "block", "block": 64, "sink_blocks": 1, "local_blocks": 1, "stride_blocks": 2}, [[0]]),
    ("varlen-g256-d64", [97, 0, 60], 256, 1, 64, {"kind": "streaming", "sink": 3, "window": 20},
     [[1], [0], [0]]),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_bf16_every_element(case):
    name, seqlens, hq, hkv, D, sparse, mask = case
    print(f"[case] {name}", flush=True)
    data = _bf16_case(7, seqlens, hq, hkv, D)
    o, lse = _run_attn(data, seqlens, mask, sparse)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], cu, mask, sparse)
    H.assert_bf16_close(o, ro, name)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=H.BF16_LSE_ATOL)


@pytest.mark.parametrize("D,hq,hkv", [(64, 8, 2), (128, 8, 2), (128, 64, 2), (64, 256, 1)])
def test_small_fp32_every_element(D, hq, hkv):
    """GQA 4, and 32 and 256 (items of 8 query tokens and of one)."""
    seqlens = [190, 67]
    sparse = {"kind": "block", "block": 64, "sink_blocks": 1, "local_blocks": 1, "stride_blocks": 2}
    mask = [[1, 0], [0, 1]] if hkv == 2 else [[1], [0]]
    data = _bf16_case(11, seqlens, hq, hkv, D, scale=1.0, dtype="f32")
    o, lse = _run_attn(data, seqlens, mask, sparse)
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], np.cumsum([0] + seqlens), mask, sparse)
    H.assert_f32_close(o, ro, f"fp32 D={D} G={hq // hkv}")
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-5)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [0.02, 0.3])
def test_explicit_softmax_scale(dtype, scale):
    """A softmax scale other than 1/sqrt(D): a flat one (0.02) and a sharp one (0.3, scores
    several times larger, so the running maximum is raised often)."""
    seqlens = [260, 0, 97]
    sparse = {"kind": "streaming", "sink": 8, "window": 64}
    mask = [[1, 0], [0, 1], [1, 1]]
    data = _bf16_case(13, seqlens, 8, 2, 128, scale=1.0, dtype=dtype)
    q, k, v = H.to_dev(data["q"]), H.to_dev(data["k"]), H.to_dev(data["v"])
    T = sum(seqlens)
    cu_np = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    l = torch.full((8, T), float("nan"), dtype=torch.float32, device=H.DEV)
    o = ext.attn_prefill(q, k, v, cu_seqlens=torch.tensor(cu_np, device=H.DEV), max_seqlen=max(seqlens),
                         head_mask=torch.tensor(mask, dtype=torch.int32, device=H.DEV), sparse=sparse,
                         softmax_scale=scale, lse=l)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], cu_np, mask, sparse, scale=scale)
    if dtype == "bf16":
        H.assert_bf16_close(H.to_f64(o), ro, f"scale {scale}")
        np.testing.assert_allclose(H.to_f64(l), rl, rtol=0, atol=H.BF16_LSE_ATOL)
    else:
        H.assert_f32_close(H.to_f64(o), ro, f"scale {scale}")
        np.testing.assert_allclose(H.to_f64(l), rl, rtol=0, atol=1e-5)


def test_fp32_512_workload_full_size():
    w = syn.WORKLOADS["fp32-512-s4w64"]
    data = syn.make_qkv(w)
    o, lse = _run_attn(data, list(w.seqlens), syn.forced_mask(w), w.sparse)
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], w.cu_seqlens(), syn.forced_mask(w), w.sparse)
    H.assert_f32_close(o, ro, w.name)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-5)


@pytest.mark.parametrize("sparse", [
    {"kind": "streaming", "sink": 4, "window": 70},
    {"kind": "block", "block": 64, "sink_blocks": 1, "local_blocks": 2, "stride_blocks": 5},
    {"kind": "block", "block": 128, "sink_blocks": 1, "local_blocks": 8, "stride_blocks": 16},
])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_query_lse_counts_keys(sparse, dtype):
    """q = 0 makes every score 0, so exp(lse) is the number of keys each row attends."""
    seqlens = [1000, 2100]
    data = _bf16_case(3, seqlens, 8, 2, 128, dtype=dtype)
    data["q"] = np.zeros_like(data["q"])
    mask = [[1, 0], [0, 1]]
    _, lse = _run_attn(data, seqlens, mask, sparse)
    cu = np.cumsum([0] + seqlens)
    for b, n in enumerate(seqlens):
        for h in range(8):
            want = oracle.row_key_counts(n, bool(mask[b][h // 4]), sparse)
            got = np.rint(np.exp(lse[h, cu[b]:cu[b + 1]])).astype(np.int64)
            np.testing.assert_array_equal(got, want, err_msg=f"seq {b} head {h}")


def test_planted_needle():
    """A key aligned with one query and far outside its window: the full head retrieves its
    value, the streaming head's output is bit-identical to the unplanted run."""
    n, D = 2000, 128
    sparse = {"kind": "streaming", "sink": 64, "window": 256}
    data = _bf16_case(5, [n], 2, 2, D)
    i, jstar = 1900, 700
    planted = {kk: vv.copy() for kk, vv in data.items()}
    q64 = oracle.decode_bf16(data["q"][i, 0])
    k_needle = (20.0 / (D ** -0.5 * np.linalg.norm(q64))) * q64 / np.linalg.norm(q64)
    for g in range(2):
        planted["k"][jstar, g] = syn.round_bf16_bits(k_needle.astype(np.float32))
        planted["v"][jstar, g] = syn.round_bf16_bits(np.full(D, 3.0, dtype=np.float32))
    o0, _ = _run_attn(data, [n], [[1, 0]], sparse)
    o1, _ = _run_attn(planted, [n], [[1, 0]], sparse)
    ro, _ = oracle.attention(planted["q"], planted["k"], planted["v"], None, [[1, 0]], sparse, rows=[i])
    assert np.all(np.abs(o1[i, 0] - 3.0) < 0.05), o1[i, 0][:8]   # full head: the needle dominates
    H.assert_bf16_close(o1[i:i + 1], ro, "needle row")
    np.testing.assert_array_equal(o1[i, 1], o0[i, 1])            # streaming head: never sees it


def _route_dev(w, rin):
    hidden = H.to_dev(rin["hidden"])
    cu = torch.tensor(w.cu_seqlens(), dtype=torch.int32, device=H.DEV)
    logits, mask = ext.route(hidden, H.to_dev(rin["w1"]), H.to_dev(rin["w2"]), cu_seqlens=cu,
                             threshold=rin["threshold"])
    torch.cuda.synchronize()
    del hidden
    return logits.cpu().numpy().astype(np.float64), mask.cpu().numpy()


def _check_router(w, rin, logits, mask, band=1e-3):
    ref = oracle.route(rin["hidden"], w.cu_seqlens(), rin["w1"], rin["w2"], rin["threshold"])
    outside = np.abs(ref["logits"] - rin["threshold"]) >= band
    print(f"[router] {w.name} logits gpu {logits.ravel()[:8]} ref {ref['logits'].ravel()[:8]} "
          f"in-band {int((~outside).sum())}/{outside.size}", flush=True)
    np.testing.assert_array_equal(mask[outside], ref["mask"][outside])
    np.testing.assert_allclose(logits, ref["logits"], rtol=1e-3, atol=2e-6)
    assert set(np.unique(mask)) <= {0, 1}
    return ref


def _sampled_attention(w, data, mask, heads=None, lse=True):
    o, l = _run_attn(data, list(w.seqlens), mask, w.sparse, lse=lse)
    rows = H.sample_rows_global(w)
    hs = list(range(w.n_q_heads)) if heads is None else heads
    print(f"[sample] {w.name}: {len(rows)} rows x {len(hs)} heads", flush=True)
    ro, rl = oracle.attention(data["q"], data["k"], data["v"], w.cu_seqlens(), mask, w.sparse,
                              rows=rows, heads=hs, workers=16)
    H.assert_bf16_close(o[rows][:, hs], ro, f"{w.name} mask={np.asarray(mask).tolist()}")
    if lse:
        np.testing.assert_allclose(l[hs][:, rows], rl, rtol=0, atol=H.BF16_LSE_ATOL)
    return o, l


@pytest.mark.parametrize("name", ["llama8b-8k-stream-router", "llama8b-32k-block-router"])
def test_router_then_attention_full_size(name):
    w = syn.WORKLOADS[name]
    print(f"[case] {name}", flush=True)
    rin = syn.make_router_inputs(w)
    logits, mask = _route_dev(w, rin)
    _check_router(w, rin, logits, mask)
    data = syn.make_qkv(w)
    _sampled_attention(w, data, mask)


def test_router_stress_weights():
    """Larger router weights put almost no head inside the tie band, so the mask check bites."""
    w = syn.WORKLOADS["llama8b-8k-stream-router"]
    rin = syn.make_router_inputs(w, w_std=0.02 ** 0.5)
    logits, mask = _route_dev(w, rin)
    ref = _check_router(w, rin, logits, mask)
    assert (np.abs(ref["logits"]) >= 1e-3).mean() > 0.8


def test_router_boundary_pooling_and_empty_sequence():
    lens = [300, 0, 1000, 150]
    T, d = sum(lens), 512
    hidden = syn.draw_bf16_bits(21, 3, (T, d))
    w1 = syn.draw_f32(21, 4, (64, d), 0.1)
    w2 = syn.draw_f32(21, 5, (5, 64), 0.1)
    cu_np = np.cumsum([0] + lens).astype(np.int32)
    cu = torch.tensor(cu_np, device=H.DEV)
    for ph, pt in ((0, 0), (100, 100), (7, 0)):
        logits, mask = ext.route(H.to_dev(hidden), H.to_dev(w1), H.to_dev(w2), cu_seqlens=cu,
                                 pool_head=ph, pool_tail=pt)
        ref = oracle.route(hidden, cu_np, w1, w2, 0.0, pool_head=ph, pool_tail=pt)
        lg = logits.cpu().numpy()
        np.testing.assert_allclose(lg, ref["logits"], rtol=1e-4, atol=1e-6)
        outside = np.abs(ref["logits"]) >= 1e-5
        np.testing.assert_array_equal(mask.cpu().numpy()[outside], ref["mask"][outside])
        assert np.all(lg[1] == 0) and np.all(mask.cpu().numpy()[1] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_router_ragged_strips_wide_mlp(dtype):
    """d_model not a multiple of the 64-column strip (last strip partial), a router width of 200
    (several passes of the finishing step), 12 KV heads, a varlen batch; repeated calls agree
    bit for bit, also on a reused workspace that starts as 0xFF bytes."""
    lens = [777, 64, 1, 2050]
    T, d, dr, hkv = sum(lens), 1000, 200, 12
    hidden = syn.draw_bf16_bits(31, 3, (T, d))
    if dtype == "fp32":
        hidden = (hidden.astype(np.uint32) << 16).view(np.float32)
    w1 = syn.draw_f32(31, 4, (dr, d), 0.1)
    w2 = syn.draw_f32(31, 5, (hkv, dr), 0.1)
    cu_np = np.cumsum([0] + lens).astype(np.int32)
    cu = torch.tensor(cu_np, device=H.DEV)
    logits, mask = ext.route(H.to_dev(hidden), H.to_dev(w1), H.to_dev(w2), cu_seqlens=cu)
    ref = oracle.route(hidden, cu_np, w1, w2, 0.0)
    lg = logits.cpu().numpy()
    np.testing.assert_allclose(lg, ref["logits"], rtol=1e-4, atol=1e-6)
    outside = np.abs(ref["logits"]) >= 1e-5
    np.testing.assert_array_equal(mask.cpu().numpy()[outside], ref["mask"][outside])
    logits2, _ = ext.route(H.to_dev(hidden), H.to_dev(w1), H.to_dev(w2), cu_seqlens=cu)
    np.testing.assert_array_equal(lg, logits2.cpu().numpy())
    # a workspace that starts as 0xFF bytes, used twice: the per-sequence completion counts
    # inside it are cleared by each call itself
    ws = torch.full((ext.route_workspace_size(len(lens), T, d),), 255, dtype=torch.uint8, device=H.DEV)
    for _ in range(2):
        logits3, mask3 = ext.route(H.to_dev(hidden), H.to_dev(w1), H.to_dev(w2), cu_seqlens=cu,
                                   workspace=ws)
        np.testing.assert_array_equal(lg, logits3.cpu().numpy())
        np.testing.assert_array_equal(mask.cpu().numpy(), mask3.cpu().numpy())


@pytest.mark.parametrize("frac", [0.0, 0.25, 0.5, 0.75, 1.0])
def test_qwen_64k_sparse_fraction_sweep(frac):
    w = syn.WORKLOADS["qwen-64k-stream-sweep"]
    print(f"[case] {w.name} sparse fraction {frac}", flush=True)
    data = _qwen_data()
    mask = syn.sweep_mask(w.n_kv_heads, frac)
    _sampled_attention(w, data, mask, heads=H.group_edge_heads(w.n_q_heads, w.n_kv_heads))


@pytest.mark.parametrize("sparse_heads", [[2], [1, 3], [0, 2, 3]])
def test_qwen_64k_permuted_sparse_heads(sparse_heads):
    """The same sparse fractions with other KV heads sparse: the result matches the oracle, and
    every KV group whose mode is the same as in the lowest-index choice gives identical bits
    (no item depends on how the scheduler placed the others)."""
    w = syn.WORKLOADS["qwen-64k-stream-sweep"]
    print(f"[case] {w.name} sparse heads {sparse_heads}", flush=True)
    data = _qwen_data()
    mask = np.ones((1, w.n_kv_heads), dtype=np.int32)
    mask[0, sparse_heads] = 0
    low = syn.sweep_mask(w.n_kv_heads, len(sparse_heads) / w.n_kv_heads)
    o, _ = _sampled_attention(w, data, mask, heads=H.group_edge_heads(w.n_q_heads, w.n_kv_heads),
                              lse=False)
    o_low, _ = _run_attn(data, list(w.seqlens), low, w.sparse, lse=False)
    G = w.group
    same = [g for g in range(w.n_kv_heads) if mask[0, g] == low[0, g]]
    assert same, "the two choices share no KV group"
    for g in same:
        np.testing.assert_array_equal(o[:, g * G:(g + 1) * G], o_low[:, g * G:(g + 1) * G],
                                      err_msg=f"KV group {g}")


_QWEN = {}


def _qwen_data():
    if "d" not in _QWEN:
        _QWEN["d"] = syn.make_qkv(syn.WORKLOADS["qwen-64k-stream-sweep"])
    return _QWEN["d"]


def test_varlen_184k_router_then_attention():
    w = syn.WORKLOADS["varlen-4seq-184k-stream-router"]
    rin = syn.make_router_inputs(w)
    logits, mask = _route_dev(w, rin)
    _check_router(w, rin, logits, mask)
    del rin
    data = syn.make_qkv(w)
    _sampled_attention(w, data, mask, heads=H.group_edge_heads(w.n_q_heads, w.n_kv_heads))


def test_bitwise_determinism():
    w = syn.WORKLOADS["llama8b-8k-stream-router"]
    data = _bf16_case(9, [8192], 32, 8, 128)
    mask = [[1, 0, 1, 0, 0, 1, 1, 0]]
    a, la = _run_attn(data, [8192], mask, w.sparse)
    b, lb = _run_attn(data, [8192], mask, w.sparse)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def test_empty_batch_is_a_noop():
    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=H.DEV)
    k = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=H.DEV)
    o = ext.attn_prefill(q, k, k, head_mask=None)
    assert o.shape == (0, 8, 128)

"""Benchmark of the Elastic Attention prefill hot path on one MI355X.

One step = the whole path for one layer on one batch of synthetic input already resident
in HBM: router (pool, MLP, threshold) -> scheduler -> hybrid-head GQA attention.
Prints ONE JSON line (rank 0) with the effective attention TFLOP/s (FLOPs counted only over
allowed score entries, 4 * head_dim per entry) over the step time, ms per layer, the
attention kernel's roofline fraction against the bf16 dense MFMA peak, and the fp64 CPU
oracle timed on a bounded row sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
DEFAULT_WORKLOAD = "llama8b-32k-block-router"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle sample time")
    p.add_argument("--no-supplements", action="store_true")
    p.add_argument("--no-scaling", action="store_true",
                   help="skip the streaming-head scaling sweeps (length and window)")
    p.add_argument("--copy-probe", action="store_true",
                   help="run one plain elementwise kernel first that reads 1 GiB and writes 1 GiB "
                        "(calibrates the HBM byte counters)")
    p.add_argument("--mask", choices=("workload", "full", "sparse"), default="workload",
                   help="head mask of the timed attention call: the workload's (router or forced), "
                        "every head full, or every head sparse (for per-case profiles)")
    p.add_argument("--window", type=int, default=0,
                   help="override the streaming window of a streaming workload (0: keep)")
    p.add_argument("--cpu-seconds-per-config", type=float, default=3.0,
                   help="oracle sample time for each of the other workload shapes (0: skip them)")
    return p.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (the hot path runs on a single device); "
              f"--gpus {args.gpus} / WORLD_SIZE {world} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import hybrid_sparse_full_elastic_amd as ext
    from synth import inputs as syn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    w = syn.WORKLOADS[args.workload]
    assert w.dtype == "bf16", "the timed workload is a bf16 layer"
    if args.window > 0:
        assert w.sparse["kind"] == "streaming", "--window applies to streaming workloads"
        w = w.with_(sparse=dict(w.sparse, window=args.window))

    def dev_t(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    t_gen = time.time()
    data = syn.make_qkv(w)
    q, k, v = dev_t(data["q"]), dev_t(data["k"]), dev_t(data["v"])
    has_router = w.router is not None
    if has_router:
        rin = syn.make_router_inputs(w)
        hidden, w1, w2 = dev_t(rin["hidden"]), dev_t(rin["w1"]), dev_t(rin["w2"])
        threshold = rin["threshold"]
        del rin
    cu = torch.tensor(w.cu_seqlens(), dtype=torch.int32, device=dev)
    T, hq, D = q.shape
    hkv = k.shape[1]
    B = w.batch
    o = torch.empty_like(q)
    logits = torch.empty((B, hkv), dtype=torch.float32, device=dev)
    mask = torch.empty((B, hkv), dtype=torch.int32, device=dev)
    if not has_router:
        fm = syn.forced_mask(w)
        mask.copy_(torch.from_numpy(fm))
    # the timed call's head mask: the router's (or the forced one), or an override
    attn_mask = {"workload": mask, "full": None,
                 "sparse": torch.zeros((B, hkv), dtype=torch.int32, device=dev)}[args.mask]
    ws_attn = torch.empty(ext.attn_workspace_size(0, B, T, hq, hkv, D), dtype=torch.uint8, device=dev)
    ws_route = torch.empty(max(1, ext.route_workspace_size(B, T, w.router["d_model"]) if has_router else 1),
                           dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t_gen
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if has_router:
            if ev is not None:
                ev[0].record(stream)
            ext.route(hidden, w1, w2, cu_seqlens=cu, threshold=threshold, logits=logits, mask=mask,
                      workspace=ws_route)
        if ev is not None:
            ev[1].record(stream)
        ext.attn_prefill(q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen, head_mask=attn_mask,
                         sparse=w.sparse, out=o, workspace=ws_attn)
        if ev is not None:
            ev[2].record(stream)

    if args.copy_probe:
        # one streaming elementwise kernel (not the runtime's blit kernel): 1 GiB in, 1 GiB out
        src = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    attn_ms = [e[1].elapsed_time(e[2]) for e in evs]
    route_ms = [e[0].elapsed_time(e[1]) for e in evs] if has_router else [0.0]

    # work actually done, from the mask the timed call used (host closed forms)
    mask_h = (np.ones((B, hkv), dtype=np.int32) if attn_mask is None else attn_mask.cpu().numpy())
    entries = ext.attn_entries(list(w.seqlens), mask_h, hq, hkv, w.sparse)
    flops = 4 * D * entries
    dense = hq * sum(n * (n + 1) // 2 for n in w.seqlens)
    attn_avg = float(np.mean(attn_ms))
    attn_tflops = flops / (attn_avg * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12
    router_bytes = T * w.router["d_model"] * 2 if has_router else 0
    route_avg = float(np.mean(route_ms))

    rec = {
        "metric": "effective attention TFLOP/s + ms/layer, hybrid-head GQA prefill at 32K",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": w.name, "seq_lens": list(w.seqlens), "n_q_heads": hq, "n_kv_heads": hkv,
            "head_dim": D, "sparse": w.sparse,
            "router": {k2: v2 for k2, v2 in (w.router or {}).items()} if has_router else None,
            "head_mask": mask_h.tolist(),
            "mask_source": args.mask if args.mask != "workload" else ("router" if has_router else "forced"),
            "omega_msr": float((mask_h == 0).mean()),
            "omega_esr": 1.0 - entries / dense,
            "effective_flops": flops,
        },
        "breakdown": {
            "router_us": round(route_avg * 1e3, 2),
            "router_gbs": round(router_bytes / (route_avg * 1e-3) / 1e9, 1) if has_router and route_avg > 0 else None,
            "attn_ms": round(attn_avg, 4), "attn_ms_p10": round(float(np.percentile(attn_ms, 10)), 4),
            "attn_ms_p90": round(float(np.percentile(attn_ms, 90)), 4),
            "attn_tflops": round(attn_tflops, 2),
            "note": "attn_ms brackets elastic_attn_prefill = scheduler (one small kernel) + attention kernel",
        },
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(w.name)},
        "input_gen_s": round(gen_s, 2),
    }

    if not args.no_supplements:
        rec["supplements"] = supplements(ext, torch, w, q, k, v, o, cu, ws_attn, stream, args)
        if w.batch == 1:
            rec["supplements"]["deployment"] = deployment(ext, torch, w, q, k, v, o, mask, ws_attn, stream)
        if w.batch == 1:
            rec["supplements"]["static_assignment"] = static_assignment_detail(ext, torch, w, q, k, stream)
        if has_router:
            rec["supplements"]["router"] = router_detail(ext, torch, hidden, w1, w2, cu, threshold,
                                                         logits, mask.clone(), ws_route, stream)
        del q, k, v, o
        if has_router:
            del hidden
        torch.cuda.empty_cache()
        if not args.no_scaling:
            rec["supplements"]["streaming_scaling"] = streaming_scaling(ext, torch, stream)
        rec["supplements"]["reference_gemm"] = reference_gemm(torch, stream)

    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, data, mask_h, args.cpu_seconds)
        if args.cpu_seconds_per_config > 0:
            del data
            rec["cpu_baseline"]["per_config"] = cpu_per_config(w.name, args.cpu_seconds_per_config)

    print(json.dumps(rec), flush=True)


def recorded_traffic(workload):
    """HBM bytes per attention launch from the committed FETCH_SIZE / WRITE_SIZE counter
    summary, or None when the kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"attn_bf16_kernel-{workload}.pmc.txt")
    csrc = os.path.join(ROOT, "hybrid_sparse_full_elastic_amd", "csrc")
    if not os.path.exists(path):
        return None
    fields = dict(line.split(": ", 1) for line in open(path).read().splitlines()
                  if line and not line.startswith("#") and ": " in line)
    h = hashlib.sha256()
    for name in ("attn_bf16.hip", "elastic_internal.hpp", "plan.hip"):  # kernel, tiles, schedule
        h.update(open(os.path.join(csrc, name), "rb").read())
    digest = h.hexdigest()[:16]
    if fields.get("attn_source_sha256_16") != digest:
        return None
    return int(float(fields["traffic_bytes_per_launch"]))


def _time_attn(ext, torch, stream, fn, reps=10, warm=3, min_warm_ms=50.0):
    """Mean time of one call over `reps` back-to-back calls, after `warm` calls and at least
    `min_warm_ms` of warm-up work: a short call timed right after the GPU sat idle (host-side
    input generation) would otherwise be timed while the clock is still ramping up."""
    t0 = time.perf_counter()
    n = 0
    while n < warm or (time.perf_counter() - t0) * 1e3 < min_warm_ms:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # about 1 ms of GPU work ahead of the events: the calls queue up behind it, so a call of a
    # few microseconds is timed on the GPU, not at the host's launch rate
    torch.cuda._sleep(2_000_000)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def deployment(ext, torch, w, q, k, v, o, mask, ws, stream):
    """The pages' inference settings on the same 32K layer and router mask: prefill in chunks
    of 16,384 queries (each chunk over its whole prefix) against one launch, a key range
    split in two and merged by LSE, the merge kernel's bandwidth, block-granular streaming
    (block 64, 128 sink tokens, window 1024) on every head, and explicit per-head block lists."""
    from synth import inputs as syn
    T, hq, D = q.shape
    hkv = k.shape[1]
    mask_h = mask.cpu().numpy()
    ent = ext.attn_entries([T], mask_h, hq, hkv, w.sparse)
    lse = torch.empty((hq, T), dtype=torch.float32, device=q.device)
    one = _time_attn(ext, torch, stream, lambda: ext.attn_prefill(
        q, k, v, max_seqlen=T, head_mask=mask, sparse=w.sparse, out=o, lse=lse, workspace=ws))
    C = 16384

    lse_c = torch.empty((hq, C), dtype=torch.float32, device=q.device)  # [heads, chunk rows]

    def chunked():
        for c0 in range(0, T, C):
            c1 = min(T, c0 + C)
            ext.attn_prefill_kv(q[c0:c1], k[:c1], v[:c1], head_mask=mask, sparse=w.sparse,
                                out=o[c0:c1], lse=lse_c[:, :c1 - c0], workspace=ws)
    ms_chunk = _time_attn(ext, torch, stream, chunked)
    oa, ob = torch.empty_like(o), torch.empty_like(o)
    la, lb = torch.empty_like(lse), torch.empty_like(lse)

    def split():
        ext.attn_prefill_kv(q, k[:C], v[:C], q_pos=0, k_pos=0, head_mask=mask, sparse=w.sparse,
                            out=oa, lse=la, workspace=ws)
        ext.attn_prefill_kv(q, k[C:], v[C:], q_pos=0, k_pos=C, head_mask=mask, sparse=w.sparse,
                            out=ob, lse=lb, workspace=ws)
        ext.lse_merge(oa, la, ob, lb, out=o, lse_out=lse)
    ms_split = _time_attn(ext, torch, stream, split)
    ms_merge = _time_attn(ext, torch, stream, lambda: ext.lse_merge(oa, la, ob, lb, out=o, lse_out=lse))
    merge_bytes = 3 * o.numel() * o.element_size() + 3 * lse.numel() * 4
    bstream = {"kind": "block", "block": 64, "sink_blocks": 2, "local_blocks": 15, "stride_blocks": 0}
    zeros = torch.zeros((1, hkv), dtype=torch.int32, device=q.device)
    ms_bs = _time_attn(ext, torch, stream, lambda: ext.attn_prefill(
        q, k, v, max_seqlen=T, head_mask=zeros, sparse=bstream, out=o, workspace=ws))
    ent_bs = ext.attn_entries([T], [[0] * hkv], hq, hkv, bstream)
    # explicit per-head block lists shaped like a content-based selector's output (block 128:
    # the first block, the diagonal and 8% of the earlier blocks), on every head and on the
    # router's sparse heads
    sel = syn.selection_lists(70, 1, hkv, T, 128, 0.08)
    sel_dev = dict(sel, row_ptr=torch.from_numpy(sel["row_ptr"]).to(q.device),
                   col_idx=torch.from_numpy(sel["col_idx"]).to(q.device))
    ms_sel = _time_attn(ext, torch, stream, lambda: ext.attn_prefill(
        q, k, v, max_seqlen=T, head_mask=zeros, sparse=sel_dev, out=o, workspace=ws))
    ent_sel = ext.attn_entries([T], [[0] * hkv], hq, hkv, sel)
    ms_selm = _time_attn(ext, torch, stream, lambda: ext.attn_prefill(
        q, k, v, max_seqlen=T, head_mask=mask, sparse=sel_dev, out=o, workspace=ws))
    ent_selm = ext.attn_entries([T], mask_h, hq, hkv, sel)
    return {"one_launch_ms": round(one, 4),
            "chunked_16384_ms": round(ms_chunk, 4),
            "chunked_tflops": round(4 * D * ent / ms_chunk / 1e9, 2),
            "key_split_merge_ms": round(ms_split, 4),
            "lse_merge_us": round(ms_merge * 1e3, 2),
            "lse_merge_gbs": round(merge_bytes / (ms_merge * 1e-3) / 1e9, 1),
            "block_streaming_b64_s128_w1024_ms": round(ms_bs, 4),
            "block_streaming_tflops": round(4 * D * ent_bs / ms_bs / 1e9, 2),
            "block_lists_sel8_all_heads_ms": round(ms_sel, 4),
            "block_lists_sel8_all_heads_tflops": round(4 * D * ent_sel / ms_sel / 1e9, 2),
            "block_lists_sel8_router_mask_ms": round(ms_selm, 4),
            "block_lists_sel8_router_mask_tflops": round(4 * D * ent_selm / ms_selm / 1e9, 2)}


def reference_gemm(torch, stream):
    """For scale only, not part of the path: torch's bf16 matmul (the vendor GEMM library) on
    square problems on the same GPU, as a practical dense-MFMA rate beside the 2.5 PF datasheet
    figure."""
    out = {}
    for n in (8192, 16384):
        a = torch.randn((n, n), device="cuda:0").to(torch.bfloat16)
        b = torch.randn((n, n), device="cuda:0").to(torch.bfloat16)
        ms = _time_attn(None, torch, stream, lambda: torch.matmul(a, b), reps=10 if n == 8192 else 4)
        out[f"matmul_bf16_{n}_ms"] = round(ms, 4)
        out[f"matmul_bf16_{n}_tflops"] = round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1)
        del a, b
    torch.cuda.empty_cache()
    return out


def static_assignment_detail(ext, torch, w, q, k, stream):
    """The pages' static baseline (appendix C.1): retrieval scores of the layer's last token on
    a 64-token needle (reads every key once: HBM-bound) and the ranking of 32 layers x the KV
    heads by those scores."""
    T, hq, D = q.shape
    hkv = k.shape[1]
    nd = torch.tensor([[T // 2, T // 2 + 64]], dtype=torch.int32, device=q.device)
    ws = torch.empty(ext.retrieval_workspace_size(1, T, hq), dtype=torch.uint8, device=q.device)
    ms = _time_attn(ext, torch, stream, lambda: ext.retrieval_scores(q, k, nd, workspace=ws))
    nbytes = T * hkv * D * k.element_size() + hq * D * q.element_size()
    scores = torch.rand((32, hkv), generator=torch.Generator(device=q.device).manual_seed(5),
                        device=q.device)
    out = torch.empty((32, hkv), dtype=torch.int32, device=q.device)
    ms_a = _time_attn(ext, torch, stream, lambda: ext.static_assignment(scores, 0.375, out=out))
    return {"retrieval_scores_us": round(ms * 1e3, 2),
            "retrieval_scores_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "assignment_32x%d_us" % hkv: round(ms_a * 1e3, 2)}


def router_detail(ext, torch, hidden, w1, w2, cu, threshold, logits, mask, ws, stream, reps=10):
    """Router alone with the 256 MB MALL flushed before every call (a 1 GiB read in between,
    outside the timed events, so the cache holds clean unrelated lines): mean pooling over all
    rows, and boundary pooling of the first and last 100 rows (appendix H.4 of the summary)."""
    scratch = torch.zeros(1 << 28, dtype=torch.float32, device=hidden.device)
    out = {}
    T, d = hidden.shape
    for name, ph, pt in (("mean_pool", 0, 0), ("boundary_pool_100_100", 100, 100)):
        times = []
        for r in range(reps + 2):
            scratch.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            ext.route(hidden, w1, w2, cu_seqlens=cu, threshold=threshold, pool_head=ph, pool_tail=pt,
                      logits=logits, mask=mask, workspace=ws)
            b.record(stream)
            torch.cuda.synchronize()
            if r >= 2:
                times.append(a.elapsed_time(b) * 1e3)
        us = float(np.median(times))
        rows = T if ph == 0 else min(T, (ph + pt) * (cu.numel() - 1))
        out[name] = {"us_median": round(us, 2), "hbm_gbs": round(rows * d * 2 / (us * 1e-6) / 1e9, 1)}
    del scratch
    return out


def supplements(ext, torch, w, q, k, v, o, cu, ws, stream, args):
    """Full-heads-only attention on the same tensors (the 50%-of-peak target shape)."""
    T, hq, D = q.shape
    hkv = k.shape[1]
    ms = _time_attn(ext, torch, stream, lambda: ext.attn_prefill(
        q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen, head_mask=None, sparse=None, out=o, workspace=ws))
    flops = 4 * D * ext.attn_entries(list(w.seqlens), None, hq, hkv, None)
    out = {"full_heads_only": {"attn_ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 2),
                               "frac_bf16_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}}
    all_sparse = torch.zeros((w.batch, hkv), dtype=torch.int32, device=q.device)
    ms_s = _time_attn(ext, torch, stream, lambda: ext.attn_prefill(
        q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen, head_mask=all_sparse, sparse=w.sparse, out=o, workspace=ws))
    flops_s = 4 * D * ext.attn_entries(list(w.seqlens), all_sparse.cpu().numpy(), hq, hkv, w.sparse)
    out["sparse_heads_only"] = {"attn_ms": round(ms_s, 4), "tflops": round(flops_s / ms_s / 1e9, 2)}
    return out


def streaming_scaling(ext, torch, stream):
    """All heads streaming (32 query / 8 KV heads, D 128): time per allowed entry across
    sequence lengths (sink 128 + window 1024), and time against window size at 64K.  Inputs
    are prefixes of one seeded 131K-token draw."""
    from synth import inputs as syn
    nmax, hq, hkv, D = 131072, 32, 8, 128
    dev = "cuda:0"

    def dev_bits(seed, tag, shape):
        x = syn.draw_bf16_bits(seed, tag, shape, 0.5)
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    q = dev_bits(7, 0, (nmax, hq, D))
    k = dev_bits(7, 1, (nmax, hkv, D))
    v = dev_bits(7, 2, (nmax, hkv, D))
    o = torch.empty_like(q)
    ws = torch.empty(ext.attn_workspace_size(0, 1, nmax, hq, hkv, D), dtype=torch.uint8, device=dev)
    sparse_mask = torch.zeros((1, hkv), dtype=torch.int32, device=dev)

    def run(n, sparse):
        qs, ks, vs, os_ = q[:n], k[:n], v[:n], o[:n]
        ms = _time_attn(ext, torch, stream, lambda: ext.attn_prefill(
            qs, ks, vs, max_seqlen=n, head_mask=sparse_mask, sparse=sparse, out=os_, workspace=ws))
        entries = ext.attn_entries([n], [[0] * hkv], hq, hkv, sparse)
        return ms, entries

    by_len = []
    sp = {"kind": "streaming", "sink": 128, "window": 1024}
    for n in (8192, 16384, 32768, 65536, 131072):
        ms, e = run(n, sp)
        by_len.append({"n": n, "ms": round(ms, 4), "ns_per_kentry": round(ms * 1e6 / (e / 1e3), 4)})
    per = [r["ns_per_kentry"] for r in by_len]
    by_win = []
    for wdw in (512, 1024, 2048, 4096):
        ms, e = run(65536, {"kind": "streaming", "sink": 128, "window": wdw})
        by_win.append({"window": wdw, "ms": round(ms, 4)})
    ratios = [round(by_win[i + 1]["ms"] / by_win[i]["ms"], 3) for i in range(len(by_win) - 1)]
    return {"by_length_sink128_window1024": by_len,
            "time_per_entry_spread": round(max(per) / min(per) - 1.0, 4),
            "length_check_pass": max(per) / min(per) - 1.0 <= 0.20,
            "by_window_64k": by_win, "window_doubling_ratios": ratios,
            "window_check_pass": all(1.6 <= r <= 2.2 for r in ratios)}


def _host_cpu():
    """(threads the oracle uses, CPUs visible to this process, CPU model).  The oracle's pool is
    capped at 16 threads, a one-GPU share of a multi-GPU host's cores."""
    try:
        visible = len(os.sched_getaffinity(0))
    except AttributeError:
        visible = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return max(1, min(visible, 16)), visible, model


def _oracle_rows(w, data, mask_h, target_s, cores, seed0=0, rows_per=8):
    """Seeded row batches of workload w through the attention oracle until target_s of oracle
    time: returns (seconds, effective FLOPs of the sampled rows, rows)."""
    import oracle
    from synth import inputs as syn
    D = w.head_dim
    cu = w.cu_seqlens()
    elapsed, flops, nrows, seed = 0.0, 0, 0, 0
    while elapsed < target_s and seed < 64:
        rows = np.concatenate([syn.spread_rows(int(n), rows_per, (seed0 + seed) * 131 + b) + int(cu[b])
                               for b, n in enumerate(w.seqlens) if n > 0])
        t = time.time()
        oracle.attention(data["q"], data["k"], data["v"], cu, mask_h, w.sparse, rows=rows,
                         workers=cores)
        elapsed += time.time() - t
        seq_of = np.searchsorted(cu, rows, side="right") - 1
        for b in range(w.batch):
            loc = rows[seq_of == b] - cu[b]
            if len(loc) == 0:
                continue
            for g in range(w.n_kv_heads):
                cnt = oracle.row_key_counts(int(w.seqlens[b]), bool(mask_h[b, g]), w.sparse, rows=loc)
                flops += 4 * D * w.group * int(cnt.sum())
        nrows += len(rows)
        seed += 1
    return elapsed, flops, nrows


def cpu_baseline(w, data, mask_h, target_s):
    """The fp64 oracle on the host cores, on a bounded seeded row sample of the workload."""
    cores, visible, model = _host_cpu()
    elapsed, flops, nrows = _oracle_rows(w, data, mask_h, target_s, cores)
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{nrows} seeded rows x all {w.n_q_heads} query heads of {w.name} "
                      f"({elapsed:.1f} s, fp64 numpy, {cores} threads)",
            "cpu_model": model, "cpus_visible": visible}


def cpu_per_config(main_name, target_s):
    """The oracle on each of the other workload shapes, in the workload list's order: router
    (pooling, MLP, threshold) timed whole where the shape has one, attention on seeded row
    batches for about target_s, and the whole layer's oracle time extrapolated from the
    sampled rate (FLOPs over allowed entries)."""
    import oracle
    import hybrid_sparse_full_elastic_amd as ext
    from synth import inputs as syn
    cores, _, _ = _host_cpu()
    out = []
    for name in syn.WORKLOAD_ORDER:
        if name == main_name:
            continue
        w = syn.WORKLOADS[name]
        rec = {"workload": name}
        data = syn.make_qkv(w)
        if w.router is not None:
            rin = syn.make_router_inputs(w)
            t = time.time()
            r = oracle.route(rin["hidden"], w.cu_seqlens(), rin["w1"], rin["w2"], rin["threshold"])
            rec["router_s"] = round(time.time() - t, 3)
            mask = r["mask"]
            del rin
        elif w.forced_mask is not None and name != "qwen-64k-stream-sweep":
            mask = syn.forced_mask(w)
        else:
            mask = syn.sweep_mask(w.n_kv_heads, 0.5)   # the sparse-fraction sweep's middle point
        sec, flops, nrows = _oracle_rows(w, data, mask, target_s, cores, seed0=17)
        total = 4 * w.head_dim * ext.attn_entries(list(w.seqlens), mask, w.n_q_heads, w.n_kv_heads, w.sparse)
        rate = flops / sec
        rec.update({"mask": mask.tolist(), "rows_sampled": nrows, "attention_s": round(sec, 3),
                    "tflops": round(rate / 1e12, 6),
                    "attention_full_layer_s_extrapolated": round(total / rate, 1)})
        out.append(rec)
        del data
    return out


if __name__ == "__main__":
    main()

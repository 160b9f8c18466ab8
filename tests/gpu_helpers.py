"""Shared helpers of the GPU parity tests: host <-> device marshalling and error statistics."""
import numpy as np
import torch

from synth import inputs as syn

DEV = "cuda:0"
# bf16 tolerances on the output (decoded to fp64, oracle output not rounded): max-abs and
# mean-abs bound every element; the per-head relative RMS keeps the check meaningful where
# the outputs themselves are small (long, flat softmax rows).
BF16_MAX_ABS, BF16_MEAN_ABS, BF16_REL_RMS = 2e-2, 2e-3, 1e-2
# bf16 log-sum-exp (natural log): the row sum adds the weights as rounded to bf16 for the P.V
# product (round to nearest, unit roundoff 2^-8), so |d lse| <= log(1 + 2^-8) = 3.9e-3 when
# every weight of a row rounds the same way; the fp32 score, exp2 and log add below 1e-5.
BF16_LSE_ATOL = 4e-3
F32_MAX_ABS = 1e-4


def to_dev(x: np.ndarray) -> torch.Tensor:
    """uint16 arrays are bf16 bit patterns; float32 arrays stay fp32."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def qkv_dev(w: syn.Workload, data=None):
    data = data if data is not None else syn.make_qkv(w)
    return data, to_dev(data["q"]), to_dev(data["k"]), to_dev(data["v"])


def err_stats(got: np.ndarray, ref: np.ndarray) -> dict:
    """got/ref: [rows, heads, D] float64."""
    d = np.abs(got - ref)
    num = np.sqrt(((got - ref) ** 2).sum(axis=(0, 2)))
    den = np.sqrt((ref ** 2).sum(axis=(0, 2)))
    rel = num / np.maximum(den, 1e-30)
    return {"max_abs": float(d.max()), "mean_abs": float(d.mean()), "max_rel_rms": float(rel.max()),
            "ref_rms": float(np.sqrt((ref ** 2).mean()))}


def assert_bf16_close(got, ref, what=""):
    s = err_stats(got, ref)
    print(f"[parity] {what} {s}", flush=True)
    assert s["max_abs"] <= BF16_MAX_ABS, (what, s)
    assert s["mean_abs"] <= BF16_MEAN_ABS, (what, s)
    assert s["max_rel_rms"] <= BF16_REL_RMS, (what, s)
    return s


def assert_f32_close(got, ref, what=""):
    s = err_stats(got, ref)
    print(f"[parity] {what} {s}", flush=True)
    assert s["max_abs"] <= F32_MAX_ABS, (what, s)
    return s


def pattern_reach(sparse: dict) -> int:
    """Tokens a sparse row attends at most besides its own block: sink + window for streaming,
    the sink, local and diagonal blocks for the block pattern."""
    if sparse["kind"] == "streaming":
        return int(sparse["sink"]) + int(sparse["window"])
    return (int(sparse["sink_blocks"]) + int(sparse["local_blocks"]) + 1) * int(sparse["block"])


def sample_rows_global(w: syn.Workload) -> np.ndarray:
    """Sorted global token indices of the deterministic full-size sample: per sequence, the
    first 2 * reach rows (where sink and window edges move), every 16th block of 128 rows, and
    the last block."""
    cu = w.cu_seqlens()
    reach = pattern_reach(w.sparse)
    return np.concatenate([syn.sample_rows(int(n), reach) + int(cu[b]) for b, n in enumerate(w.seqlens)])


def group_edge_heads(n_q_heads: int, n_kv_heads: int) -> list:
    """The first and the last query head of every KV group."""
    G = n_q_heads // n_kv_heads
    return sorted({h for g in range(n_kv_heads) for h in (g * G, g * G + G - 1)})


def global_rows(w: syn.Workload, per_seq: int, seed: int = 0) -> np.ndarray:
    """Sorted global token indices: a seeded spread of rows per sequence (first/last included)."""
    cu = w.cu_seqlens()
    out = []
    for b, n in enumerate(w.seqlens):
        out.append(syn.spread_rows(int(n), per_seq, seed + b) + int(cu[b]))
    return np.concatenate(out)


def random_lists(seed, batch, hkv, nqb, B, density=0.3, extras=True):
    """Seeded CSR: each row lists a random subset of key blocks 0..qb (sometimes empty, sometimes
    without the diagonal, sometimes with a later block that must be ignored)."""
    rng = np.random.default_rng(seed)
    rp, ci = [0], []
    for _ in range(batch * hkv):
        for qb in range(nqb):
            kbs = set(np.nonzero(rng.random(qb + 1) < density)[0].tolist())
            if rng.random() < 0.7:
                kbs.add(qb)
            if extras and rng.random() < 0.2 and qb + 1 < nqb:
                kbs.add(qb + 1)            # a later block: ignored
            if rng.random() < 0.05:
                kbs = set()                # the block's rows see nothing
            ci.extend(sorted(kbs))
            rp.append(len(ci))
    return {"kind": "block_list", "block": B, "qblocks": nqb, "row_ptr": rp, "col_idx": ci}


def dev_lists(lists):
    d = dict(lists)
    d["row_ptr"] = torch.tensor(lists["row_ptr"], dtype=torch.int32, device=DEV)
    d["col_idx"] = torch.tensor(lists["col_idx"] if lists["col_idx"] else [0], dtype=torch.int32,
                                device=DEV)
    return d

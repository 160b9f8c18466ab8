"""Shared helpers of the GPU parity tests: host <-> device marshalling and error statistics."""
import numpy as np
import torch

from synth import inputs as syn

DEV = "cuda:0"
# bf16 tolerances on the output (decoded to fp64, oracle output not rounded): max-abs and
# mean-abs bound every element; the per-head relative RMS keeps the check meaningful where
# the outputs themselves are small (long, flat softmax rows).
BF16_MAX_ABS, BF16_MEAN_ABS, BF16_REL_RMS = 2e-2, 2e-3, 1e-2
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


def global_rows(w: syn.Workload, per_seq: int, seed: int = 0) -> np.ndarray:
    """Sorted global token indices: a seeded spread of rows per sequence (first/last included)."""
    cu = w.cu_seqlens()
    out = []
    for b, n in enumerate(w.seqlens):
        out.append(syn.spread_rows(int(n), per_seq, seed + b) + int(cu[b]))
    return np.concatenate(out)

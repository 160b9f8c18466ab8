"""Build libelastic.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m hybrid_sparse_full_elastic_amd.build`` (or ``build()`` from Python).
Objects go to ``_build/`` at the repository root; the shared library is written next to
this file as ``libelastic.so`` and replaced atomically.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libelastic.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for every device compile.  The atomic optimizer
# is off: it rewrites a one-lane atomic into a wave-level one whose result is consumed (with a
# wait on every outstanding load) right after it, which would serialise the attention prologue
# behind its work-queue claim.  The other atomics here are single-lane or go to lane-dependent
# addresses, which the optimizer does not rewrite.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain (ROCm) is required to build libelastic")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only target feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _llvm_tool(name: str) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "llvm", "bin", name)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found; the ROCm LLVM tools are required to build libelastic")
    return path


def kernel_metadata(obj: str) -> list:
    """The AMDGPU metadata (amdhsa.kernels) of the gfx950 code object inside a host object
    built by this script: its .hip_fatbin section is a clang offload bundle."""
    import tempfile
    import yaml
    with tempfile.TemporaryDirectory() as tmp:
        fat, co = os.path.join(tmp, "fatbin"), os.path.join(tmp, "device.co")
        _run([_llvm_tool("llvm-objcopy"), "-O", "binary", "--only-section=.hip_fatbin", obj, fat], False)
        _run([_llvm_tool("clang-offload-bundler"), "--type=o", "--unbundle", f"--input={fat}",
              f"--output={co}", f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}"], False)
        r = subprocess.run([_llvm_tool("llvm-readelf"), "--notes", co], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"llvm-readelf failed on {obj}: {r.stderr}")
    text = r.stdout
    begin = text.index("---")
    end = text.index("\n...", begin)
    return yaml.safe_load(text[begin:end])["amdhsa.kernels"]


def check_attn_kernargs(meta: list) -> int:
    """The bf16 attention kernels read their arguments through the kernel argument segment
    pointer, as a struct at offset 0.  Every instance must take exactly one explicit argument,
    by value, at offset 0.  Returns the number of instances checked; raises otherwise."""
    n = 0
    for k in meta:
        if "attn_bf16_kernel" not in k[".name"]:
            continue
        explicit = [a for a in k.get(".args", []) if not a[".value_kind"].startswith("hidden_")]
        if len(explicit) != 1 or explicit[0][".offset"] != 0 or explicit[0][".value_kind"] != "by_value":
            raise RuntimeError(f"{k['.name']}: kernel arguments {explicit} are not one by-value "
                               "struct at offset 0, which the kernel's argument reads assume")
        n += 1
    if n == 0:
        raise RuntimeError("no attn_bf16_kernel instance found in the code object")
    return n


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link libelastic.so. Returns the library path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with ThreadPoolExecutor(max(1, min(jobs, len(srcs)))) as ex:
        list(ex.map(lambda so: _run([cc, *HIPCC_FLAGS, "-c", so[0], "-o", so[1]], verbose),
                    zip(srcs, objs)))
    check_attn_kernargs(kernel_metadata(os.path.join(BUILD_DIR, "attn_bf16.o")))
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

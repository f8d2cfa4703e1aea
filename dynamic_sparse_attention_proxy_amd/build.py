"""Build libcrisp.so (HIP kernels + C-ABI) for gfx950 with hipcc, in-tree.

    python -m dynamic_sparse_attention_proxy_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "crisp")
LIB = os.path.join(HERE, "libcrisp.so")
SOURCES = ["route.hip", "select.hip", "jsd.hip", "attention.hip", "abi.hip"]
# per-source extra flags: the attention kernels never produce or test NaN, so max
# needs no NaN canonicalisation
EXTRA = {"attention.hip": ["-fno-honor-nans"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # exact fp32 operation order for the decision steps: no contraction
    "-ffp-contract=off",
    # no packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, obj_dir: str = OBJ, defines=()) -> str:
    out = os.path.join(obj_dir, src + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link ``out``; ``defines`` are extra -D macros."""
    obj_dir = OBJ if out == LIB else os.path.join(ROOT, "_build", os.path.basename(out) + ".obj")
    os.makedirs(obj_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

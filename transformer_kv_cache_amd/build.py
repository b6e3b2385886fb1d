"""Build libkvcache.so (HIP kernels for gfx950 + the C ABI) in the package
directory with hipcc.  Run as ``python -m transformer_kv_cache_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvcache.so")
SOURCES = ["kvc_api.hip", "kvc_append.hip", "kvc_decode.hip", "kvc_decode_mfma.hip",
           "kvc_decode_rows.hip", "kvc_prefill.hip", "kvc_dense.hip", "kvc_gemm.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: no accvgpr copies around the per-tile rescale
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, build_dir: str = BUILD_DIR, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(f"-D{d}" for d in defines), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = True, out: str = LIB, defines=(), build_dir: str = BUILD_DIR) -> str:
    """Compile every source and link `out`.  `defines` are extra -D macros
    (build-time tuning constants such as KVC_DECODE_KEYS_PER_LANE)."""
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()

"""Build librownorm.so (the HIP kernels + C ABI) for gfx950, in-tree.

    python -m row_normalization_persistent_amd.build

Every translation unit is compiled by hipcc for gfx950 only, with packed-fp32
VALU instructions disabled, then linked into one shared library next to this
file.  Object files go to ``_build/`` at the repository root.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "librownorm.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = [
    "api.hip",
    "k_fused_add_rmsnorm.hip",
    "k_rmsnorm_fwd.hip",
    "k_layernorm_fwd.hip",
    "k_norm_bwd.hip",
    "k_fused_add_rmsnorm_dyn.hip",
    "k_rmsnorm_fwd_dyn.hip",
    "k_layernorm_fwd_dyn.hip",
    "k_layernorm_bwd_dyn.hip",
    "k_rmsnorm_bwd_dyn.hip",
    "k_split.hip",
    "k_bwd_wide.hip",
    "k_stream.hip",
]

# Benchmark-only measurement kernel (not part of the normalization library):
# its own shared library, loaded by bench.py alone.
CEILING_SOURCES = ["ceiling.hip"]
CEILING_LIB_PATH = os.path.join(PKG, "libnormceiling.so")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    # keep every fp32 VALU op scalar: no packed fp32 add/mul/fma
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librownorm.so)")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(extra_flags=(), jobs: int | None = None, out_path: str | None = None,
          build_dir: str | None = None) -> str:
    """Compile every source and link the library (LIB_PATH unless out_path).
    Always rebuilds."""
    global BUILD_DIR
    out_path = out_path or LIB_PATH
    saved, BUILD_DIR = BUILD_DIR, build_dir or BUILD_DIR
    try:
        os.makedirs(BUILD_DIR, exist_ok=True)
        jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
        with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
            objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES))
    finally:
        BUILD_DIR = saved
    tmp = out_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out_path)
    return out_path


def build_ceiling() -> str:
    """Compile and link libnormceiling.so (the benchmark's same-traffic
    measurement kernel).  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [_compile(src, []) for src in CEILING_SOURCES]
    tmp = CEILING_LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, CEILING_LIB_PATH)
    return CEILING_LIB_PATH


if __name__ == "__main__":
    print(build())
    print(build_ceiling())

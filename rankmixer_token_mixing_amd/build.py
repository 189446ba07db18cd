"""Compile librankmixer.so in-tree with hipcc for gfx950.

    python -m rankmixer_token_mixing_amd.build

Every HIP source is compiled to an object (in parallel), then linked into
``rankmixer_token_mixing_amd/librankmixer.so``.  No GPU is needed: hipcc
cross-compiles the device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librankmixer.so")
SOURCES = ["abi.cpp", "kernels_rows.hip", "kernels_moe.hip", "kernels_gemm.hip", "kernels_tokproj.hip", "kernels_bwd.hip", "kernels_variants.hip", "kernels_moe_train.hip", "kernels_probe.hip",
           "kernels_gemm_defer.hip"]
ARCH = os.environ.get("RM_OFFLOAD_ARCH", "gfx950")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere in the device code
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def source_hash() -> str:
    """sha256 (first 16 hex digits) of every C/C++/HIP source and header the
    library is built from; the build bakes it into rm_version()."""
    root = os.path.dirname(PKG)
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".hpp", ".inc")))
    files.append(os.path.join(root, "include", "rankmixer.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def library_is_fresh(path: str = LIB) -> bool:
    """Whether the library at `path` exists and was built from the tree's
    current sources (its rm_version string carries their hash)."""
    if not os.path.exists(path):
        return False
    with open(path, "rb") as fh:
        return (" src " + source_hash()).encode() in fh.read()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librankmixer.so)")


# per-source flags: the deferred-epilogue GEMM keeps its accumulators in AGPRs
# that only its inline asm names, so the compiler must never spill into AGPRs
EXTRA_FLAGS = {"kernels_gemm_defer.hip": ["-mllvm", "-amdgpu-spill-vgpr-to-agpr=0"]}


def _compile(src: str, src_hash: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), f'-DRM_SRC_HASH="{src_hash}"', "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    src_hash = source_hash()
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda f: _compile(f, src_hash), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

"""Build libvq.so (gfx950) in-tree with hipcc.

    python -m gemv_bit_unpack_amd.build

Every HIP unit is compiled with ``-ffp-contract=off`` (the dequant must not fuse its
add and multiply) and with packed-fp32 VALU instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvq.so")
CEILINGS_SRC = os.path.join(PKG, "micro", "ceilings.hip")
CEILINGS_BIN = os.path.join(PKG, "micro", "vq_ceilings")
SOURCES = ["vq_host.cpp", "vq_dequant.hip", "vq_gemv.hip", "vq_gemv_sliced.hip", "vq_gemv_bucket.hip", "vq_gemm.hip", "vq_svq.hip", "vq_rht.hip",
           "vq_assign.hip", "vq_svq_gemm.hip", "vq_gemm_gather.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
HIP_ONLY = [
    "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


# Per-unit additions.  vq_assign: matrix-core results go straight to VGPRs (the VALU reads
# every one of them), instead of through the accumulation registers.
EXTRA = {"vq_assign.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON]
    if src.endswith(".hip"):
        cmd += HIP_ONLY + EXTRA.get(src, []) + ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every unit and link ``libvq.so`` next to this file.  Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    build_ceilings()
    if verbose:
        print("built", LIB)
    return LIB


def build_ceilings() -> str:
    """The hardware-ceiling microbenchmark (stream read, global and LDS gathers)."""
    tmp = CEILINGS_BIN + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-O3", "-std=c++17", *HIP_ONLY, "-o", tmp, CEILINGS_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, CEILINGS_BIN)
    return CEILINGS_BIN


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

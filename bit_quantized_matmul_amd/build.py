"""Build libbqm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: ``python -m bit_quantized_matmul_amd.build`` (also called by
``__graft_entry__.build()``).  Every source under ``csrc/`` is compiled with
hipcc for gfx950 only, then linked into ``bit_quantized_matmul_amd/libbqm.so``.
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
LIB = os.path.join(PKG, "libbqm.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # correctly rounded fp32 division (the A8 and Q4_0 encoders rely on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 instructions anywhere (hipcc's host pass warns: harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
# sources whose results must be bit-exact: no fused multiply-add contraction
EXACT = {"act_quant.hip", "cq_pack.hip", "codebook_fit.hip", "q4_0.hip"}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libbqm")
    return path


def sources() -> list[str]:
    """All HIP sources, the long compiles (GEMV kernel sets, GEMM) first."""
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    return sorted(srcs, key=lambda f: (not f.startswith("cq_gemv_i"), f != "cq_gemm.hip", f))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    flags = list(COMMON)
    if src in EXACT:
        flags.append("-ffp-contract=off")
    cmd = [hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()

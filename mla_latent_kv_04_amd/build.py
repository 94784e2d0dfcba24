"""Build the HIP library libmla_latent_kv.so for gfx950 with hipcc (in-tree).

Usage: python -m mla_latent_kv_04_amd.build   (or build() from Python).
The shared object lands in mla_latent_kv_04_amd/_lib/; object files go to
mla_latent_kv_04_amd/_build/.  Every call recompiles every source.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libmla_latent_kv.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are not used in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Keep compiler-generated MFMA accumulators in the VGPR form; the register
# allocator then places long-lived operands in AGPRs.  The two-role kernels
# (decode_h64.hip, decode_h64_fp8.hip) are the exception: their value waves
# keep their accumulators in AGPRs (AGPR form).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
SOURCES = ["kv_append.hip", "absorb_q.hip", "decode.hip", "decode_h64.hip", "decode_h64_fp8.hip",
           "decode_fp8.hip",
           "combine.hip", "out_proj.hip", "produce.hip", "prefill_mha.hip", "noalloc.hip",
           "mla_api.cpp", "produce_api.cpp"]
EXTRA = {src: VGPR_FORM for src in SOURCES
         if src.endswith(".hip") and src not in ("decode_h64.hip", "decode_h64_fp8.hip")}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MLA library)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

"""Builds libtpshard.so (HIP, gfx950) in-tree from csrc/.

    python -m tensor_transformer_layer_rank_amd.build [-j N] [--asm]

Objects go to _build/ at the repository root; the shared library is written
next to this file, where the binding loads it.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtpshard.so")
ARCH = "gfx950"

SOURCES = ["tpshard.cpp", "copy_kernels.hip", "gemm.hip", "attn_prefill.hip",
           "attn_flash.hip", "lm_argmax.hip", "norm.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libtpshard)")


FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function", "-Wno-unused-variable",
         # packed-fp32 VALU forms are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


# per-source flags: the attention kernels run one wave per SIMD and keep
# their MFMA accumulators in ordinary VGPRs (with AGPR accumulators the
# compiler copied the output tiles between the register files on every key
# tile; measured 10-20% slower)
_VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
EXTRA = {"attn_flash.hip": _VGPR_MFMA, "attn_prefill.hip": _VGPR_MFMA}


def _compile(src: str, asm: bool) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    if asm:
        s = os.path.join(BUILD, src + ".s")
        subprocess.run([hipcc(), *FLAGS, *EXTRA.get(src, []), "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", s],
                       capture_output=True, text=True, check=True)
    return obj


def build(jobs: int = 0, asm: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=0)
    ap.add_argument("--asm", action="store_true", help="also write device assembly to _build/")
    a = ap.parse_args()
    print(build(a.j, a.asm))

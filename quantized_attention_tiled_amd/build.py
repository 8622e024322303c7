"""Build libqattn.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m quantized_attention_tiled_amd.build [--jobs N] [--verbose]
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqattn.so")
SOURCES = ["qattn_abi.hip", "attn_fwd_bf16.hip", "attn_fwd_f16.hip", "attn_qbsa.hip", "quant.hip", "attn_bwd.hip",
           "mask_pack.hip"]
ARCH = "gfx950"

# Packed fp32 instructions are switched off for all device code; the host
# pass warns that it does not know the feature, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The attention kernels run two waves per SIMD (256 registers per lane) and keep every MFMA
# accumulator in ordinary VGPRs, so no accumulator is copied between register files.
SOURCE_FLAGS = {"attn_fwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
                "attn_fwd_f16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
                "attn_qbsa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
                "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c", f"-I{INCLUDE}", f"-I{CSRC}",
           *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 5, verbose: bool = False) -> str:
    """Compile every HIP source and link libqattn.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libqattn.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=5)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())

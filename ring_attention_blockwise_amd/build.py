"""Build libra.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python ring_attention_blockwise_amd/build.py

Each source is compiled with hipcc to an object in ``_build/``, in parallel,
then linked into ``ring_attention_blockwise_amd/libra.so``.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libra.so")
SOURCES = ["ra_api.cpp", "attn_step.hip", "attn_step_bf16.hip", "attn_bwd_bf16.hip", "attn_bwd_simt.hip",
           "merge_relayout.hip"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are turned off for all device code.  Code
# object v5 loads under every ROCm 7 runtime, including the one bundled with
# PyTorch, which is the runtime this library shares at run time.  MFMAs keep
# their accumulators in ordinary vector registers: kernels that run one wave
# per SIMD (512 registers) would otherwise get every MFMA in the
# accumulation-register form and copy each score tile out before the
# softmax; the accumulation registers then hold read-only MFMA operands.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mcode-object-version=5",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-Wall", "-Wno-unused-function", *DEVICE_FLAGS,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

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
# PyTorch, which is the runtime this library shares at run time.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mcode-object-version=5"]


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


def asan_runtime() -> str | None:
    """The compiler's shared AddressSanitizer runtime (to preload into the
    Python process that loads the sanitized build), or None."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    base = os.path.join(rocm, "llvm", "lib", "clang")
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        path = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(path):
            return path
    return None


def build_sanitized(verbose: bool = False) -> str:
    """A second build of the library whose host code of the C ABI (argument
    checks, index maps, ring and launch plans: ra_api.cpp) is compiled with
    AddressSanitizer and UndefinedBehaviorSanitizer, linked with the normal
    kernel objects.  Only host code is instrumented (every sanitizer flag is
    given to the host compilation alone).  Returns the path of the .so; load
    it with RA_LIBRARY set to that path and the ASan runtime preloaded."""
    objs = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "ra_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    out_dir = os.path.join(BUILD, "sanitize")
    os.makedirs(out_dir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    obj = os.path.join(out_dir, "ra_api.o")
    cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
           "-Wall", "-Wno-unused-function", *DEVICE_FLAGS, *san,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-c", os.path.join(CSRC, "ra_api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized ra_api.cpp:\n{r.stderr}")
    lib = os.path.join(out_dir, "libra.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-shared-libasan", obj, *objs, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of the sanitized library failed:\n{r.stderr}")
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

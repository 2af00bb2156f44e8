"""Build libslay.so (the HIP kernels for gfx950 and the C ABI) in-tree with hipcc.

Usage: python -m kernelized_linear_attention_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libslay.so")
SOURCES = ["slay_api.cpp", "slay_featmap.hip", "slay_chunked_generic.hip", "slay_chunked_fused.hip", "slay_chunked_wide.hip",
           "slay_decode.hip", "slay_backward.hip", "slay_backward_fused.hip", "slay_noalloc.hip"]
ARCH = os.environ.get("SLAY_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU instructions are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
          "-Wno-unused-function"] + DEVICE_FLAGS


def _hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, "-I", os.path.join(PKG, "..", "include"), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libslay.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)

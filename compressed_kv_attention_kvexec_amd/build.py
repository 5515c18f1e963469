"""Build the gfx950 HIP library libtq4.so in-tree with hipcc.

Usage: python -m compressed_kv_attention_kvexec_amd.build  (or call build())."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtq4.so")
PROBE_LIB = os.path.join(PKG, "libtq4probe.so")  # streaming-read probe (measurement support)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

PROBE_SOURCES = ["tq4_probe.hip"]
SOURCES = ["tq4_api.cpp", "tq4_codebook.cpp", "tq4_encode.hip", "tq4_decode.hip", "tq4_prefill.hip",
           "tq4_dense.hip", "tq4_pages.cpp", "tq4_int8.hip", "tq4_noalloc.hip",
           "tq4_decode_valu.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
          "-Wall", "-Wno-unused-function"]
# Kernel arguments that lead with scalars (pointers, sizes) are preloaded into scalar registers at
# wave launch, so a kernel's first memory requests do not wait for a read of its argument block.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc", "-mllvm", "-amdgpu-kernarg-preload-count=16"]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    flags = list(COMMON)
    if src.endswith(".hip"):
        flags += ["-x", "hip"] + DEVICE
        if src == "tq4_encode.hip":
            flags += ["-ffp-contract=off"]
    else:
        flags += ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]
    cmd = [HIPCC] + flags + ["-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC"] + objs + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Build libtq4.so (the attention library) and libtq4probe.so (the bandwidth probe)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(PROBE_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

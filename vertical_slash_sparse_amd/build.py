"""Build libvs.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

Usage: ``python -m vertical_slash_sparse_amd.build`` (or ``build()``).  The
library is written next to this file so it travels with the source tree.
``--sanitize`` (``build(sanitize=True)``) builds libvs_san.so instead: the
same kernels, with the host code (argument checks, workspace sizing,
launches) instrumented by AddressSanitizer and UndefinedBehaviorSanitizer;
the binding loads it when VS_SANITIZE=1, with clang's ASan runtime preloaded.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libvs.so")
LIB_SAN = os.path.join(HERE, "libvs_san.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["vs_api.hip", "vs_attn.hip", "vs_index.hip", "vs_select.hip", "vs_aggregate.hip", "vs_blocks.hip"]
ARCH = os.environ.get("VS_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed fp32 arithmetic anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# host-side instrumentation only: each sanitizer flag goes to the host pass
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(OBJDIR, src.replace(".hip", "_san.o" if sanitize else ".o"))
    cmd = ["hipcc", "-c", *HIPCC_FLAGS, *(SAN_FLAGS if sanitize else []), os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    lib = LIB_SAN if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)

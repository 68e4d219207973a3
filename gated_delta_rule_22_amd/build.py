"""Build ``libckda.so`` (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: ``python -m gated_delta_rule_22_amd.build`` (also called by the repo's
``__graft_entry__.build()``).  Sources compile in parallel to objects under
``_build/`` and link into ``gated_delta_rule_22_amd/libckda.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libckda.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "schedule.hip", "decode.hip", "fwd_f64.hip", "fwd_bf16.hip", "bwd_f64.hip"]

# Packed fp32 VALU ops stay off: the compiler is not allowed to form them.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


# Host-side AddressSanitizer + UBSan for a CPU-only check of the host code
# (argument validation, workspace layout); device code is built as usual.
SAN_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -g".split()
SAN_DIR = os.path.join(BUILD, "san")


def _compile(src: str, sanitize: bool = False) -> str:
    out = SAN_DIR if sanitize else BUILD
    obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitize else []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build the library; ``sanitize`` builds the host-sanitized copy
    ``_build/san/libckda.so`` instead (load it with CKDA_LIB and a preloaded
    clang ASan runtime)."""
    os.makedirs(SAN_DIR if sanitize else BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    lib = os.path.join(SAN_DIR, "libckda.so") if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)

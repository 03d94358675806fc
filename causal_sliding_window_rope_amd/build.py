"""Build libswa.so (the HIP kernels and their C ABI) in-tree for gfx950 with hipcc.

Usage: python -m causal_sliding_window_rope_amd.build   (or __graft_entry__.build()).
Every call recompiles. Objects go to causal_sliding_window_rope_amd/_build/, the library to
causal_sliding_window_rope_amd/libswa.so.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libswa.so")
BUILD = os.path.join(PKG, "_build")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no kernel relies on NaN semantics (masks use +-inf): lets min/max skip NaN quieting
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libswa)")


# per-file additions (later flags win): the fp8 packing keeps NaN inputs NaN; decoding returns
# NaN rows for invalid positions
FILE_FLAGS = {"fp8_pack.hip": ["-fhonor-nans"], "decode.hip": ["-fhonor-nans"]}


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o",
           obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    if os.path.exists(OUT):
        os.remove(OUT)   # a failed build must not leave an older library behind
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra or []), srcs))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])

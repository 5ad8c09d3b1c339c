"""Build libmapflow.so (HIP, gfx950) in-tree: cross_model_attention_amd/lib/libmapflow.so.

Usage: ``python cross_model_attention_amd/build.py`` (or ``__graft_entry__.build()``); run by path,
since importing the package loads the library this script replaces.  Always
recompiles every source; the objects go to ``cross_model_attention_amd/_build/``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmapflow.so")
SOURCES = ["api.hip", "compress.hip", "retrieve.hip", "dense.hip"]

ARCH = os.environ.get("MAPFLOW_ARCH", "gfx950")
FLAGS = [
    "-std=c++17", "-O3", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
    "-Wno-unused-result", "-Wno-unknown-pragmas",
    # packed fp32 VALU forms stay disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (no copies through the accumulation registers)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _hipcc() -> str:
    for cand in [os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")]:
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


# Per-source flags.  The compression kernels never see NaN from valid (finite) inputs, and
# infinities (used for masking) keep their IEEE meaning under this flag; it lets max() on MFMA
# results skip the quieting step.
SOURCE_FLAGS = {"compress.hip": ["-fno-honor-nans"]}


def _compile(src: str, extra: list[str], objdir: str) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None, out: str | None = None,
          objdir: str | None = None) -> str:
    """Compile every source and link the library (``out``: another output path, with its objects
    in ``objdir``, for a build with extra flags)."""
    lib = out or LIB
    objdir = objdir or OBJ
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    extra = list(extra or [])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, objdir), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])

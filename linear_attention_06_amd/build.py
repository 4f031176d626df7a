"""Builds the in-tree HIP library ``libgdn.so`` for gfx950 with hipcc.

Every source is compiled on each call (``python -m linear_attention_06_amd.build``
or ``__graft_entry__.build()``); the objects go to ``_build/`` and are linked into
``linear_attention_06_amd/libgdn.so`` next to this file.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdn.so")
ARCH = "gfx950"

# Packed-fp32 VALU instructions are kept out of the generated code; the host
# pass of hipcc warns that it does not know the feature, which is harmless.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Per-source flags. The matrix-core kernels keep MFMA accumulators in ordinary
# VGPRs: their results feed VALU code every chunk, and accumulation registers
# would cost a copy each way.
SOURCE_FLAGS = {name: ["-mllvm", "-amdgpu-mfma-vgpr-form"] for name in ("gdn_mfma.hip", "gdn_bwd_mfma.hip")}


def _compile(src: str, extra: list) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    return obj


def build(verbose: bool = False, extra: list | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    extra = list(extra or [])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])

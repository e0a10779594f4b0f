"""Build the gfx950 HIP library ``libconv2d_gi.so`` in-tree with hipcc.

Usage: ``python -m conv2d_backward_amd.build`` (or ``build()`` from Python).
Each source compiles to an object under ``_build/`` at the repository root,
in parallel; the objects link into ``conv2d_backward_amd/libconv2d_gi.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libconv2d_gi.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [
    "api.cpp",
    "kernels_generic.hip",
    "kernels_halo_f32.hip",
    "kernels_halo_bf16.hip",
    "kernels_img16.hip",
    "kernels_stem_f32.hip",
    "kernels_col2im_f32.hip",
    "kernels_gw_f32.hip",
    "kernels_fwd_f32.hip",
    "noalloc.hip",
    "kernels_peak.hip",
]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Werror",
          "--offload-arch=" + ARCH, "-I", INCLUDE, "-I", CSRC]
# Device code: gfx950 only; packed fp32 instructions are switched off.
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + (DEVICE if src.endswith(".hip") else []) + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the gfx950 feature name; that warning is noise.
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)

"""Compile libvsa.so (all HIP sources of this package) for gfx950, in-tree.

Usage: ``python -m video_sparse_attention_amd.build`` or ``build()`` from
Python.  Objects go to ``_build/`` at the repository root, the shared library
to ``video_sparse_attention_amd/lib/libvsa.so``.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libvsa.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unknown-pragmas",
    # no packed fp32 VALU instructions anywhere (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libvsa")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=None, build_dir: str = BUILD, lib_path: str = LIB,
          link_cmd=None) -> str:
    """Compile every HIP source with ``HIPCC_FLAGS + extra_flags`` into
    ``build_dir`` and link ``lib_path``.  ``link_cmd`` (a list ending where the
    object files go) replaces hipcc's own shared-library link, e.g. for an
    instrumented host build that links a sanitizer runtime."""
    hipcc = _hipcc()
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(os.path.dirname(lib_path), exist_ok=True)
    flags = HIPCC_FLAGS + list(extra_flags or [])
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(build_dir, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        return _run([hipcc, *flags, "-c", src, "-o", obj])

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        logs = list(ex.map(compile_one, zip(srcs, objs)))
    tmp = lib_path + ".tmp"
    if link_cmd is None:
        logs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]))
    else:
        logs.append(_run([*link_cmd, "-o", tmp, *objs]))
    os.replace(tmp, lib_path)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Compiles libgnsilu.so for gfx950 with hipcc, in-tree.

Run ``python groupnorm_silu_normalization_amd/_build.py`` (by path, so the
package -- which loads the library -- is not imported first) or call
``build()``.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgnsilu.so")
SOURCES = [os.path.join(CSRC, "gn_api.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, "gn_kernels.hpp"), os.path.join(INCLUDE, "gnsilu.h")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; set HIPCC or install ROCm")


def compile_command(out: str):
    return [
        hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        # no packed fp32 (v_pk_*_f32) instructions anywhere in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
        "-o", out, *SOURCES,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libgnsilu.so")
    # hipcc's host pass does not know the packed-fp32 feature; drop that note.
    noise = [ln for ln in res.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)

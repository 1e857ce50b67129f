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


def sanitizer_command(out: str):
    """The host-sanitizer build: host code with AddressSanitizer and
    UndefinedBehaviorSanitizer (every -fsanitize after -Xarch_host, so no
    device code is instrumented), device code unoptimised (it is never
    launched: the build serves the CPU tests of the argument checks and the
    plan)."""
    return [
        hipcc(), "--offload-arch=" + ARCH, "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
        "-fno-omit-frame-pointer", "-Xarch_device", "-O0", "-Xarch_device", "-g0",
        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=undefined",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC, "-o", out, *SOURCES,
    ]


def asan_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to preload into a
    Python that is not itself instrumented), or '' if there is none."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if cand and os.path.exists(cand):
            res = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                 capture_output=True, text=True)
            path = res.stdout.strip()
            if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    return ""


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    cmd = sanitizer_command(out)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building the host-sanitizer library")
    return out


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
    if len(sys.argv) > 2 and sys.argv[1] == "--host-sanitizers":
        print(build_host_sanitized(sys.argv[2], verbose=True))
        print("preload:", asan_runtime())
    else:
        build(verbose=True)
        print(LIB)

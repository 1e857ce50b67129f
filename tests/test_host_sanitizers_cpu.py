"""The host side of libgnsilu.so under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The library's host code (argument checks, overflow checks, the launch plans,
the scratch layout arithmetic) is rebuilt with both sanitizers on the host
side only (the device code of that build is unoptimised and never launched), and the CPU test suite runs again in a child process against it,
with the sanitizer runtime preloaded into Python: any heap or stack overflow,
use after free, signed overflow, misaligned access or invalid shift in the
host code ends the child with an error report.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHILD = "GNSILU_SANITIZER_CHILD"


def _load_build():
    import importlib.util
    path = os.path.join(ROOT, "groupnorm_silu_normalization_amd", "_build.py")
    spec = importlib.util.spec_from_file_location("_gnsilu_build_san", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.skipif(os.environ.get(CHILD) == "1", reason="inside the sanitizer run itself")
def test_cpu_suite_under_host_sanitizers(tmp_path):
    b = _load_build()
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("no hipcc")
    rt = b.asan_runtime()
    if not rt:
        pytest.skip("no AddressSanitizer runtime next to the compiler")
    lib = b.build_host_sanitized(str(tmp_path / "libgnsilu.so"))
    env = dict(os.environ)
    env.update({
        CHILD: "1",
        "GNSILU_LIBRARY": lib,
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    probe = ("import ctypes, groupnorm_silu_normalization_amd as gn; "
             "assert gn.LIB_PATH == %r; "
             "ctypes.CDLL(None).__asan_init; "
             "print('sanitized library loaded')" % lib)
    res = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0 and "sanitized library loaded" in res.stdout, res.stderr[-3000:]
    res = subprocess.run([sys.executable, "-m", "pytest", "tests", "-q", "-x", "-m", "not gpu",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=1200)
    print(res.stdout[-2000:])
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error:" not in res.stderr

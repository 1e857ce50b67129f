"""C-ABI checks that need no GPU.

* libgnsilu.so loads and exports every function include/gnsilu.h declares.
* The status matrix of the argument checks, which run before any HIP call:
  GN_INVALID_ARGUMENT for input no GroupNorm accepts, GN_UNSUPPORTED for the
  inputs the library declines (a channel count with no tile layout, C above
  GN_MAX_CHANNELS, a layout that is not channels-last -- the decline contract
  of "FLUX.2 VAE decoder fast path behind quality=high", Modifications
  section 1, over a wider supported set), GN_OK for empty input.  The
  pointers passed here are never dereferenced: every case returns before the
  library touches HIP.
* The Python binding's None contract for inputs it declines on the host.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gnsilu.h")

gn = pytest.importorskip("groupnorm_silu_normalization_amd")
from groupnorm_silu_normalization_amd import GnStatus  # noqa: E402

# Fake, 16-byte aligned, never dereferenced device addresses.
X = ctypes.c_void_p(0x10000)
Y = ctypes.c_void_p(0x20000)
I64x4 = ctypes.c_int64 * 4
I64x5 = ctypes.c_int64 * 5
# Channel counts used below that the library declines: 257 (prime), 2056
# (8*257) and 3000 (8*375) have no tile layout; 8200 and 16384 exceed
# GN_MAX_CHANNELS.


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("gn_silu_nhwc", "gn_silu_rows", "gn_silu_nhwc_strided", "gn_stats_rows",
                 "gn_apply_rows", "gn_profile_rows", "gn_status_string", "gn_silu_ndhwc",
                 "gn_silu_ndhwc_strided_dtype", "gn_plan_single_launch", "gn_silu_rows_noalloc"):
        assert must in names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    for n in names:
        assert hasattr(gn.lib, n), "symbol %s declared but not exported" % n
    out = subprocess.run(["nm", "-D", "--defined-only", gn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported


def test_device_info_rejects_bad_arguments_without_a_hip_call():
    out = (ctypes.c_int64 * 6)(*([-7] * 6))
    assert gn.gn_device_info(0, None) == GnStatus.INVALID_ARGUMENT
    assert gn.gn_device_info(-1, out) == GnStatus.INVALID_ARGUMENT
    assert list(out) == [-7] * 6


def test_status_strings_and_version():
    for s in GnStatus:
        assert gn.status_text(s).startswith("GN_" + s.name)
    assert gn.gn_version() >= 100
    assert [gn.gn_kernel_name(i).decode() for i in range(4)] == [
        "gn_partial_stats", "gn_finalize_stats", "gn_apply", "gn_strip"]
    assert gn.gn_kernel_name(4) is None and gn.gn_kernel_name(-1) is None


def rows(x=X, y=Y, N=1, L=16, C=64, G=32, eps=1e-6, silu=1):
    return gn.gn_silu_rows(x, None, None, y, N, L, C, G, eps, silu, None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(y=None), dict(N=-1), dict(L=-1), dict(C=0), dict(C=-8),
    dict(G=0), dict(G=-2), dict(C=64, G=3), dict(C=96, G=5), dict(eps=-1e-3),
    dict(eps=float("nan")), dict(eps=float("inf")), dict(silu=2), dict(silu=-1),
    dict(N=2 ** 40, L=2 ** 20, C=1024),
])
def test_invalid_arguments(kw):
    assert rows(**kw) == GnStatus.INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [
    dict(C=257, G=1), dict(C=2056, G=8), dict(C=3000, G=1), dict(C=16384, G=32),
    dict(C=8200, G=8), dict(x=ctypes.c_void_p(0x10002)), dict(y=ctypes.c_void_p(0x20008)),
])
def test_unsupported_inputs(kw):
    assert rows(**kw) == GnStatus.UNSUPPORTED


@pytest.mark.parametrize("N,L", [(0, 16), (1, 0), (0, 0)])
def test_empty_input_is_ok_without_gpu(N, L):
    assert rows(N=N, L=L) == GnStatus.OK
    assert gn.gn_silu_nhwc(X, None, None, Y, N, L, 1, 64, 32, 1e-6, 1, None) == GnStatus.OK


@pytest.mark.parametrize("dtype", [-1, 3, 7])
def test_invalid_dtype(dtype):
    assert gn.gn_silu_rows_dtype(X, None, None, Y, 1, 16, 64, 32, 1e-6, 1, dtype,
                                 None) == GnStatus.INVALID_ARGUMENT
    assert gn.gn_stats_rows_dtype(X, 1, 16, 64, 32, 1e-6, dtype, Y, Y,
                                  None) == GnStatus.INVALID_ARGUMENT


def test_dtype_entry_points_share_the_checks():
    for dt in (0, 1, 2):
        assert gn.gn_silu_rows_dtype(X, None, None, Y, 1, 16, 3000, 8, 1e-6, 1, dt,
                                     None) == GnStatus.UNSUPPORTED
        assert gn.gn_silu_ndhwc_dtype(X, None, None, Y, 1, 2, 2, 4, 3000, 8, 1e-6, 1, dt,
                                      None) == GnStatus.UNSUPPORTED
        assert gn.gn_silu_rows_dtype(X, None, None, Y, 0, 16, 64, 32, 1e-6, 1, dt,
                                     None) == GnStatus.OK
        assert gn.gn_silu_nhwc_dtype(None, None, None, Y, 1, 4, 4, 64, 32, 1e-6, 1, dt,
                                     None) == GnStatus.INVALID_ARGUMENT


@pytest.mark.parametrize("dtype", [0x40, 0x100, 0x23, 0x13, 0x33, -0x10])
def test_invalid_affine_flags(dtype):
    assert gn.gn_silu_rows_dtype(X, None, None, Y, 1, 16, 64, 32, 1e-6, 1, dtype,
                                 None) == GnStatus.INVALID_ARGUMENT
    assert gn.gn_stats_rows_dtype(X, 1, 16, 64, 32, 1e-6, dtype, Y, Y,
                                  None) == GnStatus.INVALID_ARGUMENT


def test_affine_flags_checked_before_any_hip_call():
    odd, even2 = ctypes.c_void_p(0x30001), ctypes.c_void_p(0x30002)
    for dt in (0, 1, 2):
        for af in (0, 0x10, 0x20, 0x30):
            assert gn.gn_silu_rows_dtype(X, None, None, Y, 0, 16, 64, 32, 1e-6, 1, dt | af,
                                         None) == GnStatus.OK
            # the launch plan does not depend on the type of gamma and beta
            assert gn.plan_rows(3, 1000, 320, 32, dt | af) == gn.plan_rows(3, 1000, 320, 32, dt)
        # gamma / beta misaligned for their element type: declined
        assert gn.gn_silu_rows_dtype(X, odd, None, Y, 1, 16, 64, 32, 1e-6, 1, dt | 0x20,
                                     None) == GnStatus.UNSUPPORTED
        assert gn.gn_silu_rows_dtype(X, None, odd, Y, 1, 16, 64, 32, 1e-6, 1, dt | 0x30,
                                     None) == GnStatus.UNSUPPORTED
        assert gn.gn_silu_rows_dtype(X, even2, None, Y, 1, 16, 64, 32, 1e-6, 1, dt,
                                     None) == GnStatus.UNSUPPORTED
        assert gn.gn_silu_rows_dtype(X, None, even2, Y, 1, 16, 64, 32, 1e-6, 1, dt | 0x10,
                                     None) == GnStatus.UNSUPPORTED
        assert gn.gn_apply_rows_dtype(X, Y, Y, odd, None, Y, 1, 16, 64, 32, 1, dt | 0x20,
                                      None) == GnStatus.UNSUPPORTED


def test_affine_flags_match_the_header():
    text = open(HEADER).read()
    vals = {k: int(v, 16) for k, v in re.findall(r"(GN_AFFINE_\w+) = (0x[0-9a-fA-F]+)", text)}
    assert vals["GN_AFFINE_F32"] == gn.AFFINE_FLAG[torch.float32]
    assert vals["GN_AFFINE_BF16"] == gn.AFFINE_FLAG[torch.bfloat16]
    assert vals["GN_AFFINE_F16"] == gn.AFFINE_FLAG[torch.float16]
    assert vals["GN_AFFINE_MASK"] == 0x30
    # the binding's choice of flag for weight and bias
    from groupnorm_silu_normalization_amd.binding import _affine_flag
    t = torch.zeros(4)
    assert _affine_flag(None, None) == 0
    assert _affine_flag(t, None) == 0x10
    assert _affine_flag(t.bfloat16(), t.bfloat16()) == 0x20
    assert _affine_flag(None, t.half()) == 0x30
    assert _affine_flag(t, t.bfloat16()) is None


def test_plan_uses_element_size_for_the_cache_threshold():
    # (1,512,512,512): 256 MiB in bf16/fp16 (fits the cache), 512 MiB in fp32
    assert gn.plan_rows(1, 512 * 512, 512, 32, gn.GnDtype.BF16)["apply_nontemporal_loads"] == 0
    assert gn.plan_rows(1, 512 * 512, 512, 32, gn.GnDtype.F16)["apply_nontemporal_loads"] == 0
    assert gn.plan_rows(1, 512 * 512, 512, 32, gn.GnDtype.F32)["apply_nontemporal_loads"] == 1


def test_nhwc_checks():
    f = gn.gn_silu_nhwc
    assert f(X, None, None, Y, 1, -1, 4, 64, 32, 1e-6, 1, None) == GnStatus.INVALID_ARGUMENT
    assert f(X, None, None, Y, 1, 4, -1, 64, 32, 1e-6, 1, None) == GnStatus.INVALID_ARGUMENT
    assert f(X, None, None, Y, 1, 4, 4, 2056, 8, 1e-6, 1, None) == GnStatus.UNSUPPORTED
    assert f(X, None, None, Y, 1, 2 ** 40, 2 ** 40, 8, 1, 1e-6, 1, None) == GnStatus.INVALID_ARGUMENT


def test_ndhwc_checks():
    f = gn.gn_silu_ndhwc
    for D, H, W in ((-1, 4, 4), (4, -1, 4), (4, 4, -1), (2 ** 30, 2 ** 30, 2 ** 30)):
        assert f(X, None, None, Y, 1, D, H, W, 64, 32, 1e-6, 1, None) == GnStatus.INVALID_ARGUMENT
    assert f(X, None, None, Y, 1, 2, 4, 4, 3000, 8, 1e-6, 1, None) == GnStatus.UNSUPPORTED
    assert f(X, None, None, Y, 1, 0, 4, 4, 64, 32, 1e-6, 1, None) == GnStatus.OK
    assert f(X, None, None, Y, 2, 3, 0, 4, 64, 32, 1e-6, 1, None) == GnStatus.OK


def test_ndhwc_strided_rejects_ncdhw_and_other_layouts():
    N, C, D, H, W = 2, 64, 3, 5, 7
    cl = I64x5(D * H * W * C, 1, H * W * C, W * C, C)
    ncdhw = I64x5(C * D * H * W, D * H * W, H * W, W, 1)
    swapped = I64x5(D * H * W * C, 1, W * C, D * W * C, C)  # H and D exchanged
    f = gn.gn_silu_ndhwc_strided_dtype
    for xs, ys in ((ncdhw, cl), (cl, ncdhw), (swapped, cl)):
        assert f(X, xs, None, None, Y, ys, N, D, H, W, C, 32, 1e-6, 1, 0,
                 None) == GnStatus.UNSUPPORTED
    assert f(X, ncdhw, None, None, Y, cl, N, D, H, W, C, 7, 1e-6, 1, 0,
             None) == GnStatus.INVALID_ARGUMENT
    assert f(X, None, None, None, Y, cl, N, D, H, W, C, 32, 1e-6, 1, 0,
             None) == GnStatus.INVALID_ARGUMENT
    assert f(X, cl, None, None, Y, cl, 0, D, H, W, C, 32, 1e-6, 1, 0, None) == GnStatus.OK
    # extent-1 dimensions may carry any stride
    one = I64x5(999, 1, 5, 7 * C, C)
    assert f(X, one, None, None, Y, one, 1, 1, 0, W, C, 32, 1e-6, 1, 0, None) == GnStatus.OK


def test_strided_rejects_nchw_and_other_layouts():
    N, C, H, W = 2, 64, 5, 7
    cl = I64x4(H * W * C, 1, W * C, C)
    nchw = I64x4(C * H * W, H * W, W, 1)
    padded = I64x4(H * W * C + 8, 1, W * C, C)
    f = gn.gn_silu_nhwc_strided
    assert f(X, nchw, None, None, Y, cl, N, H, W, C, 32, 1e-6, 1, None) == GnStatus.UNSUPPORTED
    assert f(X, cl, None, None, Y, nchw, N, H, W, C, 32, 1e-6, 1, None) == GnStatus.UNSUPPORTED
    assert f(X, padded, None, None, Y, cl, N, H, W, C, 32, 1e-6, 1, None) == GnStatus.UNSUPPORTED
    # argument errors take precedence over the layout
    assert f(X, nchw, None, None, Y, cl, N, H, W, C, 7, 1e-6, 1, None) == GnStatus.INVALID_ARGUMENT
    assert f(X, None, None, None, Y, cl, N, H, W, C, 32, 1e-6, 1, None) == GnStatus.INVALID_ARGUMENT
    # empty dense input: nothing to do
    assert f(X, cl, None, None, Y, cl, 0, H, W, C, 32, 1e-6, 1, None) == GnStatus.OK


def test_stats_apply_profile_argument_checks():
    assert gn.gn_stats_rows(X, 1, 16, 64, 32, 1e-6, None, Y, None) == GnStatus.INVALID_ARGUMENT
    assert gn.gn_stats_rows(X, 1, 16, 64, 32, 1e-6, Y, None, None) == GnStatus.INVALID_ARGUMENT
    assert gn.gn_stats_rows(X, 1, 16, 2056, 8, 1e-6, Y, Y, None) == GnStatus.UNSUPPORTED
    assert gn.gn_apply_rows(X, None, Y, None, None, Y, 1, 16, 64, 32, 1, None) == GnStatus.INVALID_ARGUMENT
    ms = (ctypes.c_float * 4)()
    nk = ctypes.c_int(0)
    assert gn.gn_profile_rows(X, None, None, Y, 1, 16, 64, 32, 1e-6, 1, None, 0, ms,
                              ctypes.byref(nk)) == GnStatus.INVALID_ARGUMENT


def test_binding_declines_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 64, 4, 4, dtype=torch.bfloat16).to(memory_format=torch.channels_last)
    with torch.no_grad():
        assert gn.group_norm_silu_4d(x, 32) is None
        assert gn.group_norm_silu_rows(torch.zeros(1, 16, 64, dtype=torch.bfloat16), 32) is None
        for dt in (torch.float16, torch.float32, torch.float64):
            assert gn.group_norm_silu_4d(x.to(dt), 32) is None
    with pytest.raises(ValueError):
        gn.group_norm_silu_4d(torch.zeros(2, 3, dtype=torch.bfloat16), 1)
    with pytest.raises(TypeError):
        gn.group_norm_silu_4d([1, 2, 3], 1)


def test_header_limits_match_binding():
    text = open(HEADER).read()
    assert "#define GN_MAX_CHANNELS 8192" in text
    assert gn.MAX_CHANNELS == 8192 and math.log2(gn.MAX_CHANNELS).is_integer()


def test_one_hip_runtime_whatever_the_import_order():
    """Importing the package before torch must not map a second HIP runtime."""
    code = ("import groupnorm_silu_normalization_amd, torch\n"
            "maps = open('/proc/self/maps').read()\n"
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))\n")
    out = subprocess.run(["python", "-c", code], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout.strip().splitlines()[-1]
    assert out == "1"


def noalloc(x=X, y=Y, N=1, L=16, C=64, G=32, eps=1e-6, silu=1, dtype=0):
    return gn.gn_silu_rows_noalloc(x, None, None, y, N, L, C, G, eps, silu, dtype, None)


def test_noalloc_checks_before_any_hip_call():
    """gn_silu_rows_noalloc: the argument checks of gn_silu_rows_dtype, then the
    fixed buffer's size, all before any HIP call (the fake pointers here are
    never dereferenced)."""
    assert noalloc(x=None) == GnStatus.INVALID_ARGUMENT
    assert noalloc(C=64, G=3) == GnStatus.INVALID_ARGUMENT
    assert noalloc(dtype=3) == GnStatus.INVALID_ARGUMENT
    assert noalloc(C=257, G=1) == GnStatus.UNSUPPORTED
    assert noalloc(x=ctypes.c_void_p(0x10002)) == GnStatus.UNSUPPORTED
    assert noalloc(N=0) == GnStatus.OK and noalloc(L=0) == GnStatus.OK
    # 4096 groups: the partials of 256 chunks need 8 MiB, more than the buffer
    need = gn.plan_rows(1, 65536, 4096, 4096)["scratch_bytes"]
    assert need > gn.NOALLOC_SCRATCH_BYTES
    assert noalloc(N=1, L=65536, C=4096, G=4096) == GnStatus.SCRATCH_TOO_SMALL
    # an invalid argument still wins over the size
    assert noalloc(N=1, L=65536, C=4096, G=4096, eps=-1.0) == GnStatus.INVALID_ARGUMENT


def test_noalloc_buffer_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define GN_NOALLOC_SCRATCH_BYTES \(1 << (\d+)\)", text)
    assert m and (1 << int(m.group(1))) == gn.NOALLOC_SCRATCH_BYTES
    # the decoder shapes fit
    for N, L, C, G in ((1, 4096, 128, 32), (1, 16384, 512, 32), (1, 262144, 512, 32),
                       (1, 1048576, 256, 32), (1, 1048576, 128, 32)):
        assert gn.plan_rows(N, L, C, G)["scratch_bytes"] <= gn.NOALLOC_SCRATCH_BYTES

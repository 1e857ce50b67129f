"""ctypes binding of libgnsilu.so (argument marshalling only).

Every step of the GroupNorm(+SiLU) path runs in the library's HIP kernels;
this module turns torch tensors into device pointers, sizes and the current
HIP stream, and maps status codes to Python results.  torch provides device
memory and streams, nothing else.  There is no CPU fallback: if the library
is missing, importing this module raises.

Tensor-level API (the pair of "FLUX.2 VAE decoder fast path behind
quality=high", Modifications section 1 "Kernel"):

    group_norm_silu_4d(x, num_groups, weight, bias, eps, apply_silu, out)
    group_norm_silu_rows(x, num_groups, weight, bias, eps, apply_silu, out)

and the 5-D form group_norm_silu_5d for NDHWC (channels_last_3d) tensors.
x may be bf16, fp16 or fp32 (y has the same type).  Each returns the output
tensor, or None when the input is outside the supported set so the caller
falls back: not a GPU tensor, autograd enabled, another dtype, a channel
count the library declines (GN_UNSUPPORTED: see the supported set in
gnsilu.h; every C <= 256, every multiple of 8 up to 2048 and more), not
channels-last (4-D / 5-D) / not contiguous rows, weight/bias not fp32, bf16 or
fp16 (both of one type) on the same device.  Arguments no GroupNorm accepts raise ValueError; a failed HIP
call raises RuntimeError.

The raw C entry points are re-exported under their C names (gn_silu_nhwc,
gn_silu_rows, gn_silu_nhwc_strided, gn_silu_ndhwc, gn_stats_rows,
gn_apply_rows, gn_profile_rows, gn_plan_rows, their *_dtype forms,
gn_silu_rows_noalloc, gn_kernel_name, gn_status_string, gn_version,
gn_device_info).
"""
import ctypes
import enum
import os

# torch first: its wheel bundles a HIP runtime (torch/lib/libamdhip64.so,
# soname libamdhip64.so.7).  Loaded first, it satisfies this library's
# dependency on libamdhip64.so.7 and the process holds ONE HIP runtime.  Loaded
# the other way round, the system runtime comes in first and torch then maps
# its own copy beside it, so tensors allocated by torch are unknown to the
# runtime that launches these kernels.
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
# GNSILU_LIBRARY names another build of the same library (the host-sanitizer
# build of _build.py, for the CPU tests); by default the in-tree build.
LIB_PATH = os.environ.get("GNSILU_LIBRARY") or os.path.join(_PKG, "libgnsilu.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libgnsilu.so is not built (expected at %s); build it with "
        "`python groupnorm_silu_normalization_amd/_build.py`" % LIB_PATH)

lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


if len(_hip_runtimes_mapped()) > 1:
    raise ImportError(
        "two HIP runtimes are loaded in this process (%s); import torch before any other "
        "library that links libamdhip64" % ", ".join(_hip_runtimes_mapped()))

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_f32 = ctypes.c_float
_int = ctypes.c_int
_i64x4 = ctypes.c_int64 * 4
_i64x5 = ctypes.c_int64 * 5

lib.gn_silu_nhwc.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32, _int, _vp]
lib.gn_silu_rows.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _int, _vp]
_i64p = ctypes.POINTER(ctypes.c_int64)
lib.gn_silu_nhwc_strided.argtypes = [_vp, _i64p, _vp, _vp, _vp, _i64p, _i64, _i64, _i64, _i64,
                                     _i64, _f32, _int, _vp]
lib.gn_stats_rows.argtypes = [_vp, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp]
lib.gn_apply_rows.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp]
lib.gn_profile_rows.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _int, _vp,
                                _int, ctypes.POINTER(_f32), ctypes.POINTER(_int)]
lib.gn_silu_nhwc_dtype.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32, _int,
                                   _int, _vp]
lib.gn_silu_rows_dtype.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _int, _int,
                                   _vp]
lib.gn_silu_rows_noalloc.argtypes = lib.gn_silu_rows_dtype.argtypes
lib.gn_noalloc_scratch.argtypes = [_int, ctypes.POINTER(_vp), ctypes.POINTER(ctypes.c_int64)]
lib.gn_silu_nhwc_strided_dtype.argtypes = [_vp, _i64p, _vp, _vp, _vp, _i64p, _i64, _i64, _i64,
                                           _i64, _i64, _f32, _int, _int, _vp]
lib.gn_silu_ndhwc.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _f32, _int,
                              _vp]
lib.gn_silu_ndhwc_dtype.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _f32,
                                    _int, _int, _vp]
lib.gn_silu_ndhwc_strided_dtype.argtypes = [_vp, _i64p, _vp, _vp, _vp, _i64p, _i64, _i64, _i64,
                                            _i64, _i64, _i64, _f32, _int, _int, _vp]
lib.gn_conv3x3_nhwc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _int, _vp, _vp, _vp, _vp, _i64,
                                 _i64, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp]
lib.gn_conv3x3_plan.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _i64p]
lib.gn_conv3x3_pack_weights.argtypes = [_vp, _vp, _i64, _i64, _vp]
lib.gn_conv3x3_nhwc_packed.argtypes = lib.gn_conv3x3_nhwc.argtypes
lib.gn_stats_rows_dtype.argtypes = [_vp, _i64, _i64, _i64, _i64, _f32, _int, _vp, _vp, _vp]
lib.gn_apply_rows_dtype.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int,
                                    _int, _vp]
lib.gn_profile_rows_dtype.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _int,
                                      _int, _vp, _int, ctypes.POINTER(_f32),
                                      ctypes.POINTER(_int)]
lib.gn_plan_rows_dtype.argtypes = [_i64, _i64, _i64, _i64, _int, _i64p]
lib.gn_plan_single_launch.argtypes = [_i64, _i64, _i64, _i64, _int, _i64p]
for _name in ("gn_silu_nhwc", "gn_silu_rows", "gn_silu_nhwc_strided", "gn_stats_rows",
              "gn_apply_rows", "gn_profile_rows", "gn_silu_nhwc_dtype", "gn_silu_rows_dtype",
              "gn_silu_nhwc_strided_dtype", "gn_stats_rows_dtype", "gn_apply_rows_dtype",
              "gn_profile_rows_dtype", "gn_plan_rows_dtype", "gn_silu_ndhwc",
              "gn_silu_ndhwc_dtype", "gn_silu_ndhwc_strided_dtype", "gn_conv3x3_nhwc",
              "gn_conv3x3_plan", "gn_conv3x3_pack_weights", "gn_conv3x3_nhwc_packed",
              "gn_silu_rows_noalloc", "gn_plan_single_launch", "gn_noalloc_scratch"):
    getattr(lib, _name).restype = _int
lib.gn_plan_rows.argtypes = [_i64, _i64, _i64, _i64, _i64p]
lib.gn_plan_rows.restype = _int
lib.gn_kernel_name.argtypes = [_int]
lib.gn_kernel_name.restype = ctypes.c_char_p
lib.gn_status_string.argtypes = [_int]
lib.gn_status_string.restype = ctypes.c_char_p
lib.gn_version.argtypes = []
lib.gn_version.restype = _int
lib.gn_device_info.argtypes = [_int, _i64p]
lib.gn_device_info.restype = _int

# C entry points under their own names.
gn_silu_nhwc = lib.gn_silu_nhwc
gn_silu_rows = lib.gn_silu_rows
gn_silu_nhwc_strided = lib.gn_silu_nhwc_strided
gn_stats_rows = lib.gn_stats_rows
gn_apply_rows = lib.gn_apply_rows
gn_profile_rows = lib.gn_profile_rows
gn_kernel_name = lib.gn_kernel_name
gn_plan_rows = lib.gn_plan_rows
gn_silu_nhwc_dtype = lib.gn_silu_nhwc_dtype
gn_silu_rows_dtype = lib.gn_silu_rows_dtype
gn_silu_rows_noalloc = lib.gn_silu_rows_noalloc
gn_noalloc_scratch = lib.gn_noalloc_scratch
gn_silu_nhwc_strided_dtype = lib.gn_silu_nhwc_strided_dtype
gn_silu_ndhwc = lib.gn_silu_ndhwc
gn_silu_ndhwc_dtype = lib.gn_silu_ndhwc_dtype
gn_silu_ndhwc_strided_dtype = lib.gn_silu_ndhwc_strided_dtype
gn_conv3x3_nhwc = lib.gn_conv3x3_nhwc
gn_conv3x3_plan = lib.gn_conv3x3_plan
gn_conv3x3_pack_weights = lib.gn_conv3x3_pack_weights
gn_conv3x3_nhwc_packed = lib.gn_conv3x3_nhwc_packed
gn_stats_rows_dtype = lib.gn_stats_rows_dtype
gn_apply_rows_dtype = lib.gn_apply_rows_dtype
gn_profile_rows_dtype = lib.gn_profile_rows_dtype
gn_plan_rows_dtype = lib.gn_plan_rows_dtype
gn_plan_single_launch = lib.gn_plan_single_launch
gn_status_string = lib.gn_status_string
gn_version = lib.gn_version
gn_device_info = lib.gn_device_info

MAX_CHANNELS = 8192
NOALLOC_SCRATCH_BYTES = 1 << 20   # GN_NOALLOC_SCRATCH_BYTES


class GnDtype(enum.IntEnum):
    BF16 = 0
    F16 = 1
    F32 = 2


_TORCH_DTYPE = {torch.bfloat16: GnDtype.BF16, torch.float16: GnDtype.F16,
                torch.float32: GnDtype.F32}


def dtype_code(dt):
    """gn_dtype of a torch dtype, or None if the library does not take it."""
    return _TORCH_DTYPE.get(dt)


# Element type of gamma and beta, or-ed into the dtype argument (GN_AFFINE_*).
AFFINE_FLAG = {torch.float32: 0x10, torch.bfloat16: 0x20, torch.float16: 0x30}


def _affine_flag(weight, bias):
    """GN_AFFINE_* value for weight and bias, 0 when both are None, None when
    their types differ."""
    types = {p.dtype for p in (weight, bias) if p is not None}
    if len(types) > 1:
        return None
    return AFFINE_FLAG[types.pop()] if types else 0


def _affine_arg(weight, bias):
    f = _affine_flag(weight, bias)
    if f is None:
        raise TypeError("weight and bias must have the same dtype")
    return f


class GnStatus(enum.IntEnum):
    OK = 0
    UNSUPPORTED = 1
    INVALID_ARGUMENT = 2
    DEVICE_ERROR = 3
    SCRATCH_TOO_SMALL = 4


def status_text(code: int) -> str:
    return lib.gn_status_string(int(code)).decode()


def _torch():
    return torch


def _stream_handle(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _affine_ok(p, C, device, name):
    """None -> fine (absent); returns False when unsupported; raises if invalid."""
    torch = _torch()
    if p is None:
        return True
    if not isinstance(p, torch.Tensor):
        raise TypeError("%s must be a tensor or None" % name)
    if p.numel() != C:
        raise ValueError("%s must have C=%d elements, got %d" % (name, C, p.numel()))
    if p.dtype not in AFFINE_FLAG or p.device != device or not p.is_contiguous():
        return False
    return True


def _common_checks(x, weight, bias, C):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    if x.device.type != "cuda" or torch.version.hip is None:
        return False
    if torch.is_grad_enabled():
        return False
    if dtype_code(x.dtype) is None:
        return False
    if C > MAX_CHANNELS:
        return False
    if not _affine_ok(weight, C, x.device, "weight") or not _affine_ok(bias, C, x.device, "bias"):
        return False
    return _affine_flag(weight, bias) is not None


def _result(code, out):
    if code == GnStatus.OK:
        return out
    if code == GnStatus.UNSUPPORTED:
        return None
    if code == GnStatus.INVALID_ARGUMENT:
        raise ValueError(status_text(code))
    raise RuntimeError(status_text(code))


def _check_groups(C, num_groups):
    if not isinstance(num_groups, int) or num_groups <= 0 or C % num_groups != 0:
        raise ValueError("num_groups=%r must be a positive divisor of C=%d" % (num_groups, C))


def group_norm_silu_4d(x, num_groups, weight=None, bias=None, eps=1e-6, apply_silu=True,
                       out=None):
    """GroupNorm(+SiLU) of a channels-last tensor of logical shape (N, C, H, W)."""
    torch = _torch()
    if isinstance(x, torch.Tensor) and x.dim() != 4:
        raise ValueError("group_norm_silu_4d expects a 4-D tensor, got %d-D" % x.dim())
    N, C, H, W = x.shape if isinstance(x, torch.Tensor) else (0, 0, 0, 0)
    if not _common_checks(x, weight, bias, C):
        return None
    _check_groups(C, num_groups)
    if not x.is_contiguous(memory_format=torch.channels_last):
        return None
    if out is None:
        out = torch.empty_like(x, memory_format=torch.channels_last)
    elif out.shape != x.shape or out.dtype != x.dtype or out.device != x.device:
        raise ValueError("out must match x in shape, dtype and device")
    code = lib.gn_silu_nhwc_strided_dtype(
        _ptr(x), _i64x4(*x.stride()), _ptr(weight), _ptr(bias), _ptr(out), _i64x4(*out.stride()),
        N, H, W, C, num_groups, float(eps), 1 if apply_silu else 0,
        dtype_code(x.dtype) | _affine_flag(weight, bias), _stream_handle(x))
    return _result(code, out)


def group_norm_silu_5d(x, num_groups, weight=None, bias=None, eps=1e-6, apply_silu=True,
                       out=None):
    """GroupNorm(+SiLU) of a channels_last_3d tensor of logical shape (N, C, D, H, W)."""
    torch = _torch()
    if isinstance(x, torch.Tensor) and x.dim() != 5:
        raise ValueError("group_norm_silu_5d expects a 5-D tensor, got %d-D" % x.dim())
    N, C, D, H, W = x.shape if isinstance(x, torch.Tensor) else (0, 0, 0, 0, 0)
    if not _common_checks(x, weight, bias, C):
        return None
    _check_groups(C, num_groups)
    if not x.is_contiguous(memory_format=torch.channels_last_3d):
        return None
    if out is None:
        out = torch.empty_like(x, memory_format=torch.channels_last_3d)
    elif out.shape != x.shape or out.dtype != x.dtype or out.device != x.device:
        raise ValueError("out must match x in shape, dtype and device")
    code = lib.gn_silu_ndhwc_strided_dtype(
        _ptr(x), _i64x5(*x.stride()), _ptr(weight), _ptr(bias), _ptr(out), _i64x5(*out.stride()),
        N, D, H, W, C, num_groups, float(eps), 1 if apply_silu else 0,
        dtype_code(x.dtype) | _affine_flag(weight, bias), _stream_handle(x))
    return _result(code, out)


def group_norm_silu_rows(x, num_groups, weight=None, bias=None, eps=1e-6, apply_silu=True,
                         out=None):
    """GroupNorm(+SiLU) of contiguous rows of shape (N, L, C), C innermost."""
    torch = _torch()
    if isinstance(x, torch.Tensor) and x.dim() != 3:
        raise ValueError("group_norm_silu_rows expects a 3-D (N, L, C) tensor, got %d-D" % x.dim())
    N, L, C = x.shape if isinstance(x, torch.Tensor) else (0, 0, 0)
    if not _common_checks(x, weight, bias, C):
        return None
    _check_groups(C, num_groups)
    if not x.is_contiguous():
        return None
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    elif (out.shape != x.shape or out.dtype != x.dtype or out.device != x.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor matching x")
    code = lib.gn_silu_rows_dtype(_ptr(x), _ptr(weight), _ptr(bias), _ptr(out), N, L, C,
                                  num_groups, float(eps), 1 if apply_silu else 0,
                                  dtype_code(x.dtype) | _affine_flag(weight, bias),
                                  _stream_handle(x))
    return _result(code, out)


def group_stats_rows(x, num_groups, eps=1e-6):
    """Per-(n, g) fp32 mean and rstd of contiguous (N, L, C) rows (steps one and two)."""
    torch = _torch()
    N, L, C = x.shape
    mean = torch.empty((N, num_groups), dtype=torch.float32, device=x.device)
    rstd = torch.empty_like(mean)
    code = lib.gn_stats_rows_dtype(_ptr(x), N, L, C, num_groups, float(eps),
                                   _dtype_arg(x), _ptr(mean), _ptr(rstd), _stream_handle(x))
    r = _result(code, (mean, rstd))
    return r


def apply_rows(x, mean, rstd, weight=None, bias=None, apply_silu=True, out=None):
    """Step three alone on contiguous (N, L, C) rows, given per-(n, g) mean/rstd."""
    torch = _torch()
    N, L, C = x.shape
    G = mean.shape[-1]
    if out is None:
        out = torch.empty_like(x)
    code = lib.gn_apply_rows_dtype(_ptr(x), _ptr(mean), _ptr(rstd), _ptr(weight), _ptr(bias),
                                   _ptr(out), N, L, C, G, 1 if apply_silu else 0,
                                   _dtype_arg(x) | _affine_arg(weight, bias), _stream_handle(x))
    return _result(code, out)


PLAN_FIELDS = ("slots", "tiles", "full", "tpc1", "K1", "tpc2", "K2", "scratch_bytes",
               "apply_nontemporal_loads", "W", "A", "T", "stats_plain_tail", "late_finalize",
               "threads")


def _dtype_arg(x):
    code = dtype_code(x.dtype)
    if code is None:
        raise TypeError("unsupported dtype %s" % x.dtype)
    return int(code)


def plan_rows(N, L, C, G, dtype=GnDtype.BF16):
    """The library's launch plan for a rows shape (dict), or None if declined."""
    buf = (_i64 * len(PLAN_FIELDS))()
    code = lib.gn_plan_rows_dtype(N, L, C, G, int(dtype), buf)
    r = _result(code, True)
    if r is None:
        return None
    return dict(zip(PLAN_FIELDS, list(buf)))


SINGLE_LAUNCH_FIELDS = ("single_launch", "groups_per_workgroup", "pieces_per_row", "workgroups",
                        "threads", "pieces_per_lane")


def plan_single_launch(N, L, C, G, dtype=GnDtype.BF16):
    """Whether (and how) a rows shape runs as one launch (dict), or None if declined."""
    buf = (_i64 * 6)()
    code = lib.gn_plan_single_launch(N, L, C, G, int(dtype), buf)
    r = _result(code, True)
    if r is None:
        return None
    return dict(zip(SINGLE_LAUNCH_FIELDS, list(buf)))


def profile_rows(x, num_groups, weight, bias, eps, apply_silu, out, iters):
    """Mean per-kernel milliseconds over `iters` full calls (events around each launch)."""
    N, L, C = x.shape
    ms = (_f32 * 4)()
    nk = _int(0)
    code = lib.gn_profile_rows_dtype(_ptr(x), _ptr(weight), _ptr(bias), _ptr(out), N, L, C,
                                     num_groups, float(eps), 1 if apply_silu else 0,
                                     _dtype_arg(x) | _affine_arg(weight, bias),
                                     _stream_handle(x), int(iters), ms,
                                     ctypes.byref(nk))
    if code != GnStatus.OK:
        _result(code, None)
        raise RuntimeError("profiling declined: " + status_text(code))
    # a negative slot is a kernel not launched for this shape (finalize fused
    # into the statistics kernel)
    return {lib.gn_kernel_name(i).decode(): float(ms[i]) for i in range(nk.value) if ms[i] >= 0}


class PackedConv3x3Weight:
    """A (Co, Ci, 3, 3) bf16 weight packed once into the library's fragment
    order (gn_conv3x3_pack_weights), for repeated convolutions."""

    def __init__(self, data, Co, Ci, device):
        self.data, self.Co, self.Ci, self.device = data, Co, Ci, device
        self.shape = (Co, Ci, 3, 3)
        self.dtype = _torch().bfloat16


def pack_conv3x3_weight(weight):
    """Packs a channels_last (Co, Ci, 3, 3) bf16 weight; None if declined."""
    torch = _torch()
    if (weight.dim() != 4 or tuple(weight.shape[2:]) != (3, 3) or weight.dtype != torch.bfloat16
            or weight.device.type != "cuda"
            or not weight.is_contiguous(memory_format=torch.channels_last)):
        return None
    Co, Ci = weight.shape[0], weight.shape[1]
    packed = torch.empty(Co * 9 * Ci, dtype=torch.bfloat16, device=weight.device)
    code = lib.gn_conv3x3_pack_weights(_ptr(weight), _ptr(packed), Ci, Co,
                                       _stream_handle(weight))
    if _result(code, True) is None:
        return None
    return PackedConv3x3Weight(packed, Co, Ci, weight.device)


def conv3x3(x, weight, bias=None, *, norm=None, apply_silu=False, residual=None,
            next_groups=None, next_eps=1e-6, out=None):
    """3x3 convolution (padding 1, stride 1) of a channels-last bf16 tensor,
    with the GroupNorm(+SiLU) of its input in the prologue and, optionally,
    the statistics of its output for the next GroupNorm (gn_conv3x3_nhwc).

    x: (N, Ci, H, W) bf16, channels_last.  weight: (Co, Ci, 3, 3) bf16 in
    channels_last memory format (element [co, ci, kh, kw] at
    ((co*3 + kh)*3 + kw)*Ci + ci), or a ``PackedConv3x3Weight``.  bias: fp32 (Co,) or None.  norm: None, or
    (mean, rstd, gamma, beta) with fp32 mean/rstd of shape (N, G) (as from
    ``group_stats_rows``) and fp32 gamma/beta of shape (Ci,) or None.
    residual: (N, Co, H, W) bf16 channels_last or None.  next_groups: G2 for
    the output statistics, or None.

    Returns z, or (z, mean2, rstd2) when next_groups is given; None when the
    library declines the input (the caller falls back).
    """
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError("conv3x3 expects a 4-D (N, Ci, H, W) tensor")
    N, Ci, H, W = x.shape
    packed = isinstance(weight, PackedConv3x3Weight)
    if tuple(weight.shape[1:]) != (Ci, 3, 3):
        raise ValueError("weight must have shape (Co, Ci, 3, 3)")
    Co = weight.shape[0]
    if (x.device.type != "cuda" or torch.is_grad_enabled() or x.dtype != torch.bfloat16
            or weight.dtype != torch.bfloat16 or weight.device != x.device):
        return None
    if not x.is_contiguous(memory_format=torch.channels_last):
        return None
    if not packed and not weight.is_contiguous(memory_format=torch.channels_last):
        return None
    if bias is not None and (bias.dtype != torch.float32 or bias.numel() != Co
                             or bias.device != x.device):
        return None
    if residual is not None:
        if (tuple(residual.shape) != (N, Co, H, W) or residual.dtype != torch.bfloat16
                or not residual.is_contiguous(memory_format=torch.channels_last)):
            return None
    nm = nr = ga = be = None
    G = 0
    if norm is not None:
        nm, nr, ga, be = norm
        G = nm.shape[-1]
        for t in (nm, nr):
            if t.dtype != torch.float32 or t.device != x.device or not t.is_contiguous():
                return None
        if not _affine_ok(ga, Ci, x.device, "gamma") or not _affine_ok(be, Ci, x.device, "beta"):
            return None
        if any(t is not None and t.dtype != torch.float32 for t in (ga, be)):
            return None  # the convolution's prologue takes fp32 gamma and beta
    if out is None:
        out = torch.empty((N, Co, H, W), dtype=torch.bfloat16, device=x.device,
                          memory_format=torch.channels_last)
    m2 = r2 = None
    G2 = 0
    if next_groups is not None:
        G2 = int(next_groups)
        m2 = torch.empty((N, G2), dtype=torch.float32, device=x.device)
        r2 = torch.empty_like(m2)
    fn = lib.gn_conv3x3_nhwc_packed if packed else lib.gn_conv3x3_nhwc
    code = fn(
        _ptr(x), _ptr(nm), _ptr(nr), _ptr(ga), _ptr(be), G, 1 if apply_silu else 0,
        _ptr(weight.data if packed else weight), _ptr(bias), _ptr(residual), _ptr(out), N, H, W,
        Ci, Co, G2, float(next_eps), _ptr(m2), _ptr(r2), _stream_handle(x))
    r = _result(code, out)
    if r is None:
        return None
    return (out, m2, r2) if next_groups is not None else out


CONV_PLAN_FIELDS = ("tiles_h", "tiles_w", "nb", "xcd_map", "blocks", "grid", "wn")


def conv_plan(N, H, W, Ci, Co, G2=0):
    """The library's launch shape for gn_conv3x3_nhwc (dict), or None if declined."""
    buf = (_i64 * len(CONV_PLAN_FIELDS))()
    r = _result(lib.gn_conv3x3_plan(N, H, W, Ci, Co, G2, buf), True)
    return None if r is None else dict(zip(CONV_PLAN_FIELDS, list(buf)))


DEVICE_INFO_FIELDS = ("compute_units", "engine_clock_khz", "memory_clock_khz",
                      "memory_bus_bits", "memory_bytes", "wavefront")


def device_info(device=0):
    """gn_device_info of HIP device `device` as a dict (raises RuntimeError
    when the query fails)."""
    out = (ctypes.c_int64 * len(DEVICE_INFO_FIELDS))()
    code = lib.gn_device_info(int(device), out)
    if code != GnStatus.OK:
        raise RuntimeError(status_text(code))
    return dict(zip(DEVICE_INFO_FIELDS, (int(v) for v in out)))

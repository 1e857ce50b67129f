"""fp64 CPU oracle for channels-last GroupNorm(+SiLU) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it and never falls back to it.

The arithmetic lives in ``gn_oracle.c`` (plain C, fp64, two-pass); this module
only marshals numpy arrays through ctypes.  The definition it follows is the
channels-last GroupNorm with optional SiLU of "FLUX.2 VAE decoder fast path
behind quality=high", Modifications section 1 "Kernel": per-(batch, group)
statistics over (N, L, C) rows with C innermost, affine transform, optional
SiLU.

Parity status of each function (what pins it, see ``tests/test_oracle_pins.py``):
  * ``group_stats`` -- pinned: exact rational brute force, library
    GroupNorm/LayerNorm/InstanceNorm, invariants.
  * ``gn_silu`` -- pinned: exact-arithmetic brute force (Fraction/Decimal),
    torch's fp64 CPU ``group_norm`` + ``silu``, LayerNorm (G=1) and
    InstanceNorm (G=C) identities, closed-form cases, invariants; for fp16
    and fp32 inputs, torch's fp64 ``group_norm`` on the same values.
  * ``widen`` -- pinned exhaustively: all 65536 bf16 and all 65536 fp16 bit
    patterns against numpy's own conversions.
  * ``conv3x3`` -- pinned: torch's fp64 CPU ``conv2d`` (padding 1), exact
    rational brute force on tiny inputs, identity / shift / linearity
    invariants that fix the tap orientation, the padding and the weight
    layout.
  * ``conv3x3_at`` -- the same per-pixel sum as ``conv3x3`` at selected
    pixels; pinned equal to ``conv3x3`` there.
  * ``gn_silu_conv3x3`` -- composition of the pinned ``gn_silu``,
    ``conv3x3`` and ``group_stats`` (fp64 input), nothing else.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgnoracle.so")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# Input dtypes: uint16 arrays are bf16 bit patterns, float16 and float32
# arrays are IEEE binary16 / binary32 values (float64 for the statistics of
# an fp64 tensor).
_DTYPE_CODE = {np.dtype(np.uint16): 0, np.dtype(np.float16): 1, np.dtype(np.float32): 2,
               np.dtype(np.float64): 3}


def _as_input(x):
    x = np.ascontiguousarray(x)
    if x.dtype not in _DTYPE_CODE:
        raise TypeError("oracle input must be bf16 bits (uint16), float16, float32 or float64")
    return x, _DTYPE_CODE[x.dtype]


class Oracle:
    """ctypes front end of one build of ``gn_oracle.c``."""

    def __init__(self, lib_path):
        lib = ctypes.CDLL(lib_path)
        i64 = ctypes.c_int64
        vp = ctypes.c_void_p
        ci = ctypes.c_int
        lib.gno_group_stats_dt.argtypes = [vp, ci, i64, i64, i64, i64, vp, vp]
        lib.gno_group_stats_dt.restype = ci
        lib.gno_gn_silu_dt.argtypes = [vp, ci, vp, vp, i64, i64, i64, i64, ctypes.c_double,
                                       ci, vp, vp, vp, vp]
        lib.gno_gn_silu_dt.restype = ci
        lib.gno_widen.argtypes = [vp, ci, i64, vp]
        lib.gno_widen.restype = ci
        lib.gno_max_threads.argtypes = []
        lib.gno_max_threads.restype = ctypes.c_int
        lib.gno_set_threads.argtypes = [ctypes.c_int]
        lib.gno_set_threads.restype = None
        lib.gno_conv3x3_nhwc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp]
        lib.gno_conv3x3_nhwc.restype = ci
        lib.gno_conv3x3_nhwc_at.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i64,
                                            vp, vp]
        lib.gno_conv3x3_nhwc_at.restype = ci
        self.lib = lib
        self.path = lib_path

    def max_threads(self) -> int:
        return int(self.lib.gno_max_threads())

    def set_threads(self, n: int) -> None:
        self.lib.gno_set_threads(int(n))

    def conv3x3(self, inp, wt, bias, N, H, W, Ci, Co, res=None, return_abs=False):
        """3x3 convolution, zero padding 1, stride 1, NHWC, in fp64.

        inp: [N, H, W, Ci] values (any input dtype; widened exactly);
        wt: [Co, 3, 3, Ci] values; bias: [Co] or None; res: [N, H, W, Co] or
        None (added to the output).  Returns out [N, H, W, Co] float64, and
        with ``return_abs`` also the per-output sum of absolute terms.
        """
        def f64(a, n, name):
            if a is None:
                return None
            a = self.widen(a).reshape(-1) if np.asarray(a).dtype != np.float64 else \
                np.ascontiguousarray(a, np.float64).reshape(-1)
            if a.size != n:
                raise ValueError("%s has %d elements, expected %d" % (name, a.size, n))
            return a
        i64 = f64(inp, N * H * W * Ci, "inp")
        w64 = f64(wt, Co * 9 * Ci, "wt")
        b64 = f64(bias, Co, "bias")
        r64 = f64(res, N * H * W * Co, "res")
        out = np.empty(max(N * H * W * Co, 1), np.float64)
        mag = np.empty_like(out) if return_abs else None
        rc = self.lib.gno_conv3x3_nhwc(_ptr(i64), _ptr(w64), _ptr(b64), _ptr(r64), N, H, W, Ci,
                                       Co, _ptr(out), _ptr(mag))
        if rc != 0:
            raise ValueError("oracle rejected conv shape")
        out = out[: N * H * W * Co].reshape(N, H, W, Co)
        if return_abs:
            return out, mag[: N * H * W * Co].reshape(N, H, W, Co)
        return out

    def conv3x3_at(self, inp, wt, bias, N, H, W, Ci, Co, pix, res=None):
        """The convolution at selected output pixels: pix holds linear pixel
        indices (n*H + h)*W + w; returns (out, mag), each [len(pix), Co]."""
        def f64(a, n):
            if a is None:
                return None
            a = np.ascontiguousarray(a)
            a = a.reshape(-1).astype(np.float64) if a.dtype == np.float64 else \
                self.widen(a).reshape(-1)
            if a.size != n:
                raise ValueError("size mismatch")
            return a
        i64 = f64(inp, N * H * W * Ci)
        w64 = f64(wt, Co * 9 * Ci)
        b64 = f64(bias, Co)
        r64 = f64(res, N * H * W * Co)
        pix = np.ascontiguousarray(pix, np.int64)
        out = np.empty((max(pix.size, 1), Co), np.float64)
        mag = np.empty_like(out)
        rc = self.lib.gno_conv3x3_nhwc_at(_ptr(i64), _ptr(w64), _ptr(b64), _ptr(r64), N, H, W,
                                          Ci, Co, _ptr(pix), pix.size, _ptr(out), _ptr(mag))
        if rc != 0:
            raise ValueError("oracle rejected conv shape or pixel list")
        return out[: pix.size], mag[: pix.size]

    def gn_silu_conv3x3(self, x, gamma, beta, G, eps, apply_silu, wt, bias, N, H, W, Ci, Co,
                        res=None, G2=None):
        """conv3x3(GroupNorm(+SiLU)(x)) + bias (+ res), in fp64, plus the
        per-output magnitude sums and, when G2 is given, the fp64 mean and
        biased variance of each of the output's G2 groups per sample.

        Returns (z [N,H,W,Co], mag [N,H,W,Co], mean2 [N,G2] or None,
        var2 [N,G2] or None).
        """
        y = self.gn_silu(x, gamma, beta, N, H * W, Ci, G, eps, apply_silu)
        z, mag = self.conv3x3(y, wt, bias, N, H, W, Ci, Co, res=res, return_abs=True)
        mean2 = var2 = None
        if G2 is not None:
            mean2, var2 = self.group_stats(z, N, H * W, Co, G2)
        return z, mag, mean2, var2

    def widen(self, x):
        """The oracle's own fp64 widening of each input element."""
        x, code = _as_input(x)
        out = np.empty(max(x.size, 1), np.float64)
        if self.lib.gno_widen(_ptr(x), code, x.size, _ptr(out)) != 0:
            raise ValueError("bad dtype")
        return out[: x.size].reshape(x.shape)

    def group_stats(self, x_bits, N, L, C, G):
        """fp64 mean and biased variance per (n, g); arrays of shape (N, G)."""
        x, code = _as_input(x_bits)
        if x.size != N * L * C:
            raise ValueError("x has %d elements, expected N*L*C = %d" % (x.size, N * L * C))
        mean = np.empty(max(N * G, 1), np.float64)
        var = np.empty(max(N * G, 1), np.float64)
        rc = self.lib.gno_group_stats_dt(_ptr(x), code, N, L, C, G, _ptr(mean), _ptr(var))
        if rc != 0:
            raise ValueError("oracle rejected shape N=%d L=%d C=%d G=%d" % (N, L, C, G))
        return mean[: N * G].reshape(N, G), var[: N * G].reshape(N, G)

    def gn_silu(self, x_bits, gamma, beta, N, L, C, G, eps, apply_silu,
                out_dtype=np.float64, return_stats=False):
        """GroupNorm(+SiLU) of dense [N, L, C] input, computed in fp64.

        The input is bf16 bits (uint16), float16 or float32.  ``out_dtype``
        float64 returns the fp64 result; float32 returns it rounded once to
        fp32 (for the largest shapes, to halve host memory).  gamma/beta are
        float32 arrays of length C, or None (ones / zeros).
        """
        x, code = _as_input(x_bits)
        if x.size != N * L * C:
            raise ValueError("x has %d elements, expected N*L*C = %d" % (x.size, N * L * C))
        g = None if gamma is None else np.ascontiguousarray(gamma, np.float32)
        b = None if beta is None else np.ascontiguousarray(beta, np.float32)
        for name, a in (("gamma", g), ("beta", b)):
            if a is not None and a.size != C:
                raise ValueError("%s must have C=%d entries" % (name, C))
        out = np.empty(max(N * L * C, 1), np.dtype(out_dtype))
        mean = np.empty(max(N * G, 1), np.float64)
        var = np.empty(max(N * G, 1), np.float64)
        o64 = out if out.dtype == np.float64 else None
        o32 = out if out.dtype == np.float32 else None
        if o64 is None and o32 is None:
            raise TypeError("out_dtype must be float64 or float32")
        rc = self.lib.gno_gn_silu_dt(_ptr(x), code, _ptr(g), _ptr(b), N, L, C, G, float(eps),
                                     1 if apply_silu else 0, _ptr(o64), _ptr(o32),
                                     _ptr(mean), _ptr(var))
        if rc != 0:
            raise ValueError("oracle rejected arguments N=%d L=%d C=%d G=%d eps=%r"
                             % (N, L, C, G, eps))
        y = out[: N * L * C].reshape(N, L, C)
        if return_stats:
            return y, mean[: N * G].reshape(N, G), var[: N * G].reshape(N, G)
        return y


_default = None


def _get():
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _default = Oracle(_LIB_PATH)
    return _default


def max_threads() -> int:
    return _get().max_threads()


def set_threads(n: int) -> None:
    _get().set_threads(n)


def widen(x):
    return _get().widen(x)


def conv3x3(inp, wt, bias, N, H, W, Ci, Co, res=None, return_abs=False):
    return _get().conv3x3(inp, wt, bias, N, H, W, Ci, Co, res=res, return_abs=return_abs)


def conv3x3_at(inp, wt, bias, N, H, W, Ci, Co, pix, res=None):
    return _get().conv3x3_at(inp, wt, bias, N, H, W, Ci, Co, pix, res=res)


def gn_silu_conv3x3(x, gamma, beta, G, eps, apply_silu, wt, bias, N, H, W, Ci, Co, res=None,
                    G2=None):
    return _get().gn_silu_conv3x3(x, gamma, beta, G, eps, apply_silu, wt, bias, N, H, W, Ci, Co,
                                  res=res, G2=G2)


def group_stats(x_bits, N, L, C, G):
    return _get().group_stats(x_bits, N, L, C, G)


def gn_silu(x_bits, gamma, beta, N, L, C, G, eps, apply_silu, out_dtype=np.float64,
            return_stats=False):
    return _get().gn_silu(x_bits, gamma, beta, N, L, C, G, eps, apply_silu,
                          out_dtype=out_dtype, return_stats=return_stats)

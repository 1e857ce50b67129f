"""Pins of the oracle's 3x3 convolution and of its fp64-input statistics.

The convolution is the decoder's Conv2d(3x3, padding 1) of ResnetBlock2D
("FLUX.2 VAE decoder fast path behind quality=high", Modifications section 2);
its definition is the deep-learning cross-correlation with zero padding.  The
pins fix it from outside the oracle:

* torch's own fp64 CPU ``conv2d`` (a library routine) on random shapes, with
  bias and an added residual;
* exact arithmetic: small-integer inputs, where every fp64 sum is exact, against
  a brute-force sum written with Python integers;
* invariants that separate the plausible mistakes: the centre tap as identity,
  a single off-centre tap as a shift with zero fill (tap orientation and
  padding), a channel-permuting tap (weight layout [Co][3][3][Ci]), linearity;
* the magnitude sum equals the convolution of absolute values;
* the statistics of an fp64 tensor against numpy's mean / variance.
"""
import numpy as np
import pytest


def _torch_conv(x, w, b, res):
    torch = pytest.importorskip("torch")
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)            # NHWC -> NCHW
    wt = torch.from_numpy(w).permute(0, 3, 1, 2)            # [Co,3,3,Ci] -> [Co,Ci,3,3]
    bt = None if b is None else torch.from_numpy(b)
    out = torch.nn.functional.conv2d(xt, wt, bt, padding=1).permute(0, 2, 3, 1).numpy()
    return out if res is None else out + res


@pytest.mark.parametrize("N,H,W,Ci,Co,bias,res", [
    (2, 5, 7, 3, 4, True, False), (1, 9, 4, 8, 16, True, True), (3, 1, 6, 2, 5, False, True),
    (1, 6, 1, 32, 3, True, False), (2, 2, 2, 1, 1, False, False), (1, 8, 8, 16, 8, True, True),
])
def test_conv_against_torch_fp64(oracle, N, H, W, Ci, Co, bias, res):
    rng = np.random.default_rng(N * 1000 + H * 100 + W * 10 + Ci + Co)
    x = rng.standard_normal((N, H, W, Ci))
    w = rng.standard_normal((Co, 3, 3, Ci))
    b = rng.standard_normal(Co) if bias else None
    r = rng.standard_normal((N, H, W, Co)) if res else None
    got = oracle.conv3x3(x, w, b, N, H, W, Ci, Co, res=r)
    ref = _torch_conv(x, w, b, r)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_conv_exact_integer_bruteforce(oracle):
    N, H, W, Ci, Co = 1, 3, 4, 2, 2
    rng = np.random.default_rng(7)
    x = rng.integers(-5, 6, (N, H, W, Ci))
    w = rng.integers(-3, 4, (Co, 3, 3, Ci))
    b = rng.integers(-9, 10, Co)
    want = np.zeros((N, H, W, Co), dtype=object)
    for h in range(H):
        for ww in range(W):
            for co in range(Co):
                acc = int(b[co])
                for kh in range(3):
                    for kw in range(3):
                        ih, iw = h + kh - 1, ww + kw - 1
                        if 0 <= ih < H and 0 <= iw < W:
                            for ci in range(Ci):
                                acc += int(w[co, kh, kw, ci]) * int(x[0, ih, iw, ci])
                want[0, h, ww, co] = acc
    got = oracle.conv3x3(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64),
                         N, H, W, Ci, Co)
    assert np.array_equal(got, want.astype(np.float64))


def _delta(Co, Ci, kh, kw, perm=None):
    w = np.zeros((Co, 3, 3, Ci))
    for co in range(Co):
        ci = co if perm is None else perm[co]
        w[co, kh, kw, ci] = 1.0
    return w


def test_conv_centre_tap_is_identity(oracle):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 4, 5, 3))
    got = oracle.conv3x3(x, _delta(3, 3, 1, 1), None, 2, 4, 5, 3, 3)
    assert np.array_equal(got, x)


@pytest.mark.parametrize("kh,kw", [(0, 0), (0, 2), (2, 1), (1, 0), (2, 2)])
def test_conv_off_centre_tap_is_a_shift_with_zero_fill(oracle, kh, kw):
    """out[h, w] = in[h + kh - 1, w + kw - 1], zero outside the image."""
    rng = np.random.default_rng(kh * 3 + kw)
    N, H, W, C = 1, 4, 6, 2
    x = rng.standard_normal((N, H, W, C))
    got = oracle.conv3x3(x, _delta(C, C, kh, kw), None, N, H, W, C, C)
    want = np.zeros_like(x)
    for h in range(H):
        for w in range(W):
            ih, iw = h + kh - 1, w + kw - 1
            if 0 <= ih < H and 0 <= iw < W:
                want[0, h, w] = x[0, ih, iw]
    assert np.array_equal(got, want)


def test_conv_weight_layout_maps_input_to_output_channels(oracle):
    """wt[co, kh, kw, ci]: output channel co reads input channel perm[co]."""
    rng = np.random.default_rng(3)
    N, H, W, Ci, Co = 1, 3, 3, 4, 3
    perm = [2, 0, 3]
    x = rng.standard_normal((N, H, W, Ci))
    got = oracle.conv3x3(x, _delta(Co, Ci, 1, 1, perm), None, N, H, W, Ci, Co)
    assert np.array_equal(got, x[..., perm])


def test_conv_is_linear_and_adds_bias_and_residual(oracle):
    rng = np.random.default_rng(4)
    N, H, W, Ci, Co = 1, 5, 4, 3, 2
    x1, x2 = rng.standard_normal((2, N, H, W, Ci))
    w = rng.standard_normal((Co, 3, 3, Ci))
    b = rng.standard_normal(Co)
    r = rng.standard_normal((N, H, W, Co))
    f = lambda x, bb=None, rr=None: oracle.conv3x3(x, w, bb, N, H, W, Ci, Co, res=rr)
    np.testing.assert_allclose(f(2.0 * x1 - x2), 2.0 * f(x1) - f(x2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f(x1, b, r), f(x1) + b + r, rtol=1e-12, atol=1e-12)


def test_conv_magnitude_sum_is_conv_of_absolute_values(oracle):
    rng = np.random.default_rng(5)
    N, H, W, Ci, Co = 2, 4, 3, 5, 3
    x = rng.standard_normal((N, H, W, Ci))
    w = rng.standard_normal((Co, 3, 3, Ci))
    b = rng.standard_normal(Co)
    r = rng.standard_normal((N, H, W, Co))
    z, mag = oracle.conv3x3(x, w, b, N, H, W, Ci, Co, res=r, return_abs=True)
    want = oracle.conv3x3(np.abs(x), np.abs(w), np.abs(b), N, H, W, Ci, Co, res=np.abs(r))
    np.testing.assert_allclose(mag, want, rtol=1e-12, atol=1e-12)
    assert np.all(mag >= np.abs(z) - 1e-12)


def test_group_stats_of_fp64_input(oracle):
    rng = np.random.default_rng(6)
    N, L, C, G = 2, 37, 12, 3
    z = rng.standard_normal((N, L, C)) * 3.0 + 1.5
    mean, var = oracle.group_stats(z.reshape(-1).copy(), N, L, C, G)
    zg = z.reshape(N, L, G, C // G).transpose(0, 2, 1, 3).reshape(N, G, -1)
    np.testing.assert_allclose(mean, zg.mean(axis=2), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(var, zg.var(axis=2), rtol=1e-12, atol=1e-13)


def test_composition_is_conv_of_gn_silu(oracle):
    """gn_silu_conv3x3 is exactly conv3x3 of gn_silu's fp64 output plus the
    statistics of the result."""
    from gn_inputs import make_custom
    N, H, W, Ci, Co, G, G2 = 1, 6, 5, 16, 8, 4, 2
    x, gamma, beta = make_custom(N, H * W, Ci, seed=11, mean_range=(-1, 1))
    rng = np.random.default_rng(12)
    w = rng.standard_normal((Co, 3, 3, Ci)) * 0.1
    b = rng.standard_normal(Co)
    z, mag, m2, v2 = oracle.gn_silu_conv3x3(x, gamma, beta, G, 1e-6, True, w, b, N, H, W, Ci,
                                            Co, G2=G2)
    y = oracle.gn_silu(x, gamma, beta, N, H * W, Ci, G, 1e-6, True)
    assert np.array_equal(z, oracle.conv3x3(y, w, b, N, H, W, Ci, Co))
    m, v = oracle.group_stats(z.reshape(-1).copy(), N, H * W, Co, G2)
    assert np.array_equal(m2, m) and np.array_equal(v2, v)


def test_conv_at_selected_pixels_equals_full_conv(oracle):
    rng = np.random.default_rng(8)
    N, H, W, Ci, Co = 2, 5, 6, 7, 3
    x = rng.standard_normal((N, H, W, Ci))
    w = rng.standard_normal((Co, 3, 3, Ci))
    b = rng.standard_normal(Co)
    r = rng.standard_normal((N, H, W, Co))
    z, mag = oracle.conv3x3(x, w, b, N, H, W, Ci, Co, res=r, return_abs=True)
    pix = np.array([0, 5, 29, 30, 59, 17])
    zs, ms = oracle.conv3x3_at(x, w, b, N, H, W, Ci, Co, pix, res=r)
    assert np.array_equal(zs, z.reshape(-1, Co)[pix])
    assert np.array_equal(ms, mag.reshape(-1, Co)[pix])

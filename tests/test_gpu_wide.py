"""GPU parity for the widened support set, against the fp64 oracle.

The pages' kernel declines C that is not a power of two and C > 2048, and
leaves 5-D activations to an older kernel ("FLUX.2 VAE decoder fast path
behind quality=high", Modifications section 1); this library takes them
through tiles of whole rows (T = A*W*NV elements, A <= 256 active lanes).
The operation is unchanged, so the oracle and the tolerances are the ones of
the other parity tests, per element (NaN never passes):

  bf16 |y - ref| <= 1e-2 + 1.6e-2*|ref|,  fp16 1e-4 + 1e-3*|ref|,
  fp32 2e-4 + 2e-4*|ref|.

Shapes span several tiles with a ragged last tile, every layout variant
(W = 16 bytes' worth or 1; NV = 1, 2, 4; fewer than 256 active lanes), group
sizes that are not powers of two, more groups than threads (the separate
finalize), and the full-size widened workloads in the launch configuration
the benchmark times.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-2, 1.6e-2), "f16": (1e-4, 1e-3), "f32": (2e-4, 2e-4)}
CODE = {"bf16": 0, "f16": 1, "f32": 2}


@pytest.fixture(scope="module")
def gn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import groupnorm_silu_normalization_amd as g
    return g


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def to_dev(x, dev):
    """numpy input (uint16 = bf16 bits, float16, float32) -> device tensor."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(x).to(dev)


def to_host(t):
    """device tensor -> float64 numpy, flat, in memory order."""
    if t.dtype == torch.bfloat16:
        from gn_inputs import bf16_bits_to_f32
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
        return bf16_bits_to_f32(bits).astype(np.float64)
    return t.contiguous().cpu().numpy().reshape(-1).astype(np.float64)


def compare(got, ref, dtype, what):
    atol, rtol = TOL[dtype]
    ref = ref.reshape(-1).astype(np.float64)
    worst, bad, first = 0.0, 0, None
    step = 1 << 24
    for s in range(0, ref.size, step):
        g = got[s:s + step]
        r = ref[s:s + step]
        err = np.abs(g - r)
        ok = err <= atol + rtol * np.abs(r)
        nb = int(np.count_nonzero(~ok))
        if nb and first is None:
            i = int(np.flatnonzero(~ok)[0])
            first = (s + i, float(g[i]), float(r[i]))
        bad += nb
        fin = err[np.isfinite(err)]
        if fin.size:
            worst = max(worst, float(fin.max()))
    print("%s: max|y-ref|=%.3e violations=%d/%d first=%s" % (what, worst, bad, ref.size, first),
          flush=True)
    assert bad == 0, "%s: %d elements outside tolerance, first %s" % (what, bad, first)


def vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def run_rows(gn, dev, x, gamma, beta, N, L, C, G, eps, silu, dtype, inplace=False):
    xt = to_dev(x, dev)
    y = xt if inplace else torch.empty_like(xt)
    g = None if gamma is None else torch.from_numpy(gamma).to(dev)
    b = None if beta is None else torch.from_numpy(beta).to(dev)
    code = gn.gn_silu_rows_dtype(vp(xt), vp(g), vp(b), vp(y), N, L, C, G, float(eps), int(silu),
                                 CODE[dtype], stream(dev))
    assert code == gn.GnStatus.OK, gn.status_text(code)
    torch.cuda.synchronize()
    return to_host(y)


# (N, L, C, G): every case spans several tiles and ends in a ragged tile
WIDE = [
    (2, 1000, 320, 32), (1, 777, 640, 32), (2, 333, 960, 32), (1, 501, 1280, 32),
    (1, 257, 1920, 32), (2, 129, 2560, 32), (1, 65, 4096, 32), (1, 33, 8192, 32),
    (3, 501, 96, 32), (2, 999, 24, 8), (1, 4095, 3, 1), (2, 1001, 3, 3), (1, 777, 5, 5),
    (4, 31, 300, 30), (1, 7, 300, 300), (2, 171, 250, 10), (1, 100, 6144, 32),
    (1, 300, 1536, 48), (2, 31, 768, 24), (1, 5, 2560, 2560), (2, 9, 1000, 1000),
    (1, 301, 1000, 8), (2, 77, 2000, 16), (1, 500, 960, 30), (1, 500, 640, 20),
    (1, 333, 384, 12), (3, 45, 200, 40), (1, 1001, 7, 7),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("N,L,C,G", WIDE)
def test_wide_channel_counts(gn, dev, oracle, N, L, C, G, dtype):
    from gn_inputs import make_custom
    p = gn.plan_rows(N, L, C, G, CODE[dtype])
    if p is None:
        pytest.skip("outside the supported set for %s" % dtype)
    print("case N=%d L=%d C=%d G=%d %s W=%d A=%d T=%d slots=%d" % (
        N, L, C, G, dtype, p["W"], p["A"], p["T"], p["slots"]), flush=True)
    x, gamma, beta = make_custom(N, L, C, seed=7000 + C + L, mean_range=(-1, 1),
                                 std_range=(0.5, 2.0), dtype=dtype)
    y = run_rows(gn, dev, x, gamma, beta, N, L, C, G, 1e-6, 1, dtype)
    ref = oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, 1)
    compare(y, ref, dtype, "C=%d G=%d %s" % (C, G, dtype))


@pytest.mark.parametrize("C,G", [(1280, 32), (2560, 32), (320, 32), (6144, 48)])
def test_wide_cancellation_stress(gn, dev, oracle, C, G):
    """Per-channel means far from zero against a small spread: the pivot
    shift must keep the fp32 variance accurate for every layout."""
    from gn_inputs import make_custom
    N, L = 2, 777
    x, gamma, beta = make_custom(N, L, C, seed=C, mean_range=(-8, 8), std_range=(0.25, 1.0))
    y = run_rows(gn, dev, x, gamma, beta, N, L, C, G, 1e-6, 1, "bf16")
    compare(y, oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, 1), "bf16", "stress C=%d" % C)


@pytest.mark.parametrize("C,G", [(960, 32), (2560, 32), (300, 30)])
def test_wide_in_place_without_silu_or_affine(gn, dev, oracle, C, G):
    from gn_inputs import make_custom
    N, L = 2, 203
    x, _, _ = make_custom(N, L, C, seed=C + 1, affine=False)
    y = run_rows(gn, dev, x, None, None, N, L, C, G, 1e-5, 0, "bf16", inplace=True)
    compare(y, oracle.gn_silu(x, None, None, N, L, C, G, 1e-5, 0), "bf16", "in place C=%d" % C)


@pytest.mark.parametrize("C,G", [(1920, 32), (2560, 32), (1000, 1000)])
def test_wide_stats_then_apply_and_determinism(gn, dev, C, G):
    """Steps 1-2 then step 3 through the split entry points give the full
    path's output bit for bit, and repeated calls are bitwise identical."""
    from gn_inputs import make_custom
    N, L = 2, 311
    x, gamma, beta = make_custom(N, L, C, seed=C + 2)
    xt = to_dev(x, dev).reshape(N, L, C)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    with torch.no_grad():
        y1 = gn.group_norm_silu_rows(xt, G, g, b, 1e-6)
        y2 = gn.group_norm_silu_rows(xt, G, g, b, 1e-6)
        mean, rstd = gn.group_stats_rows(xt, G, 1e-6)
        y3 = gn.apply_rows(xt, mean, rstd, g, b)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))


# ------------------------------------------ 320-lane workgroups (C = 1280, 2560)
# Above 16 MiB these channel counts run steps 1 and 3 in workgroups of 320
# lanes, all busy, one 16-byte access per lane (one row of 2560 or two of 1280
# per tile).  Ragged last tiles, N = 2, all dtypes.
WIDE_APPLY = [(2, 3333, 2560, 32, "bf16"), (1, 7001, 1280, 32, "bf16"),
              (1, 7001, 1280, 32, "f16"), (2, 1777, 2560, 32, "f32"),
              (1, 6501, 1280, 16, "f32"), (1, 9001, 1280, 40, "bf16"),
              # more groups than 256 threads: whole groups per thread, separate finalize
              (1, 3333, 2560, 640, "bf16"), (1, 3333, 2560, 2560, "bf16")]


@pytest.mark.parametrize("N,L,C,G,dtype", WIDE_APPLY)
def test_wide_320_lanes(gn, dev, oracle, N, L, C, G, dtype):
    from gn_inputs import make_custom
    p = gn.plan_rows(N, L, C, G, CODE[dtype])
    print("case N=%d L=%d C=%d G=%d %s A=%d T=%d threads=%d" % (
        N, L, C, G, dtype, p["A"], p["T"], p["threads"]), flush=True)
    assert p["threads"] == 320 and p["A"] == 320 and not p["late_finalize"]
    x, gamma, beta = make_custom(N, L, C, seed=9000 + C + L, mean_range=(-1, 1),
                                 std_range=(0.5, 2.0), dtype=dtype)
    y = run_rows(gn, dev, x, gamma, beta, N, L, C, G, 1e-6, 1, dtype)
    compare(y, oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, 1), dtype,
            "320 lanes C=%d %s" % (C, dtype))
    # in place equals out of place bit for bit
    y_in = run_rows(gn, dev, x, gamma, beta, N, L, C, G, 1e-6, 1, dtype, inplace=True)
    assert np.array_equal(y_in, y)
    # steps 1-2 then step 3 given mean/rstd equal the full path bit for bit
    xt = to_dev(x, dev).reshape(N, L, C)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    with torch.no_grad():
        full = gn.group_norm_silu_rows(xt, G, g, b, 1e-6)
        mean, rstd = gn.group_stats_rows(xt, G, 1e-6)
        split = gn.apply_rows(xt, mean, rstd, g, b)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(full), to_host(split))


# ------------------------------------------------------------------ 5-D NDHWC
@pytest.mark.parametrize("N,C,D,H,W,G,dtype", [
    (1, 128, 4, 32, 32, 32, "bf16"), (2, 320, 3, 17, 19, 32, "bf16"),
    (1, 96, 5, 8, 8, 24, "f32"), (2, 64, 2, 9, 7, 8, "f16"), (1, 256, 1, 16, 16, 32, "bf16"),
])
def test_ndhwc_5d(gn, dev, oracle, N, C, D, H, W, G, dtype):
    """group_norm_silu_5d on a channels_last_3d tensor: the rows form with
    L = D*H*W, each group's statistics over all frames and positions."""
    from gn_inputs import make_custom
    L = D * H * W
    x, gamma, beta = make_custom(N, L, C, seed=500 + C + D, mean_range=(-1, 1), dtype=dtype)
    xt = to_dev(x, dev).reshape(N, D, H, W, C).permute(0, 4, 1, 2, 3)
    assert xt.is_contiguous(memory_format=torch.channels_last_3d)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    with torch.no_grad():
        y = gn.group_norm_silu_5d(xt, G, g, b, 1e-6)
    assert y is not None and y.shape == xt.shape
    assert y.is_contiguous(memory_format=torch.channels_last_3d)
    torch.cuda.synchronize()
    got = to_host(y.permute(0, 2, 3, 4, 1))
    compare(got, oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, 1), dtype,
            "5-D (%d,%d,%d,%d,%d)" % (N, C, D, H, W))


def test_ndhwc_declines_other_layouts(gn, dev):
    x = torch.randn(1, 64, 2, 4, 4, device=dev).to(torch.bfloat16)  # NCDHW-contiguous
    with torch.no_grad():
        assert gn.group_norm_silu_5d(x, 32) is None
        assert gn.group_norm_silu_5d(x.to(memory_format=torch.channels_last_3d), 32) is not None
        x3000 = torch.randn(1, 3000, 1, 2, 2, device=dev).to(torch.bfloat16)
        assert gn.group_norm_silu_5d(x3000.to(memory_format=torch.channels_last_3d), 8) is None
        with pytest.raises(ValueError):
            gn.group_norm_silu_5d(torch.zeros(2, 3, 4, 5, device=dev, dtype=torch.bfloat16), 1)


# ------------------------------------------------- full-size widened workloads
@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_wide_workload_full_size(gn, dev, oracle, idx):
    from gn_inputs import WIDE_WORKLOADS, make_inputs
    w = WIDE_WORKLOADS[idx]
    print("case %s %s" % (w.name, w.label()), flush=True)
    x, gamma, beta = make_inputs(w)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    flat = to_dev(x, dev)
    with torch.no_grad():
        if w.D == 1:
            xt = flat.reshape(w.N, w.H, w.W, w.C).permute(0, 3, 1, 2)
            y = gn.group_norm_silu_4d(xt, w.G, g, b, w.eps, apply_silu=w.apply_silu)
            got = y.permute(0, 2, 3, 1)
        else:
            xt = flat.reshape(w.N, w.D, w.H, w.W, w.C).permute(0, 4, 1, 2, 3)
            y = gn.group_norm_silu_5d(xt, w.G, g, b, w.eps, apply_silu=w.apply_silu)
            got = y.permute(0, 2, 3, 4, 1)
    assert y is not None
    torch.cuda.synchronize()
    got = to_host(got)
    del flat, xt, y
    ref = oracle.gn_silu(x, gamma, beta, w.N, w.L, w.C, w.G, w.eps, w.apply_silu,
                         out_dtype=np.float32)
    compare(got, ref, "bf16", w.name)

"""GPU parity: the HIP path against the fp64 oracle, element by element.

Tolerance (per element, NaN never passes):  |y - ref| <= 1e-2 + 1.6e-2*|ref|.
The GPU output is bf16 (relative rounding <= 2^-9 = 1.95e-3) computed from
fp32 statistics; the bound leaves room for the rounding of t = x*scale+shift
and of SiLU but fails any dropped term, wrong group or wrong pivot.

The five decoder shapes run at full size twice: through the tensor-level
group_norm_silu_4d (whose channels-last view goes to gn_silu_nhwc_strided_dtype)
and through the C entry gn_silu_nhwc itself, the call the benchmark times, in
the same launch configuration (the plan depends on the shape only).
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-2, 1.6e-2


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import groupnorm_silu_normalization_amd as gn
    return gn


@pytest.fixture(scope="module")
def gn():
    return _gpu()


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def to_dev_bits(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def from_dev_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def compare(y_bits, ref, what):
    """Element-wise tolerance check; returns (max abs err, violations)."""
    from gn_inputs import bf16_bits_to_f32
    ref = ref.reshape(-1)
    worst, bad, first = 0.0, 0, None
    step = 1 << 24
    for s in range(0, ref.size, step):
        got = bf16_bits_to_f32(y_bits[s:s + step]).astype(np.float64)
        r = ref[s:s + step].astype(np.float64)
        err = np.abs(got - r)
        ok = err <= ATOL + RTOL * np.abs(r)
        nb = int(np.count_nonzero(~ok))
        if nb and first is None:
            i = int(np.flatnonzero(~ok)[0])
            first = (s + i, float(got[i]), float(r[i]))
        bad += nb
        finite = err[np.isfinite(err)]
        if finite.size:
            worst = max(worst, float(finite.max()))
    print("%s: max|y-ref|=%.3e violations=%d/%d first=%s" % (what, worst, bad, ref.size, first),
          flush=True)
    assert bad == 0, "%s: %d elements outside tolerance, first %s" % (what, bad, first)
    return worst


def run_rows(gn, dev, x_bits, gamma, beta, N, L, C, G, eps, silu, inplace=False):
    x = to_dev_bits(x_bits, dev)
    y = x if inplace else torch.empty_like(x)
    g = None if gamma is None else torch.from_numpy(gamma).to(dev)
    b = None if beta is None else torch.from_numpy(beta).to(dev)
    code = gn.gn_silu_rows(vp(x), vp(g), vp(b), vp(y), N, L, C, G, float(eps), int(silu),
                           stream(dev))
    assert code == gn.GnStatus.OK, gn.status_text(code)
    torch.cuda.synchronize()
    return from_dev_bits(y)


# ---------------------------------------------------------------- workloads
@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_decoder_workload_full_size(gn, dev, oracle, idx):
    from gn_inputs import WORKLOADS, make_inputs
    w = WORKLOADS[idx]
    print("case %s %s" % (w.name, w.label()), flush=True)
    x_bits, gamma, beta = make_inputs(w)
    x = to_dev_bits(x_bits, dev).reshape(w.N, w.H, w.W, w.C).permute(0, 3, 1, 2)
    assert x.is_contiguous(memory_format=torch.channels_last)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    with torch.no_grad():
        y = gn.group_norm_silu_4d(x, w.G, g, b, w.eps, apply_silu=w.apply_silu)
    assert y is not None and y.is_contiguous(memory_format=torch.channels_last)
    torch.cuda.synchronize()
    y_bits = from_dev_bits(y.permute(0, 2, 3, 1))
    del x, y
    ref = oracle.gn_silu(x_bits, gamma, beta, w.N, w.L, w.C, w.G, w.eps, w.apply_silu,
                         out_dtype=np.float32)
    compare(y_bits, ref, w.name)


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_decoder_workload_through_gn_silu_nhwc(gn, dev, oracle, idx):
    """The C entry gn_silu_nhwc, called directly with device pointers and the
    current stream exactly as the benchmark calls it, at full size."""
    from gn_inputs import WORKLOADS, make_inputs
    w = WORKLOADS[idx]
    print("case gn_silu_nhwc %s %s" % (w.name, w.label()), flush=True)
    x_bits, gamma, beta = make_inputs(w)
    x = to_dev_bits(x_bits, dev)
    y = torch.empty_like(x)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    code = gn.gn_silu_nhwc(vp(x), vp(g), vp(b), vp(y), w.N, w.H, w.W, w.C, w.G, float(w.eps),
                           int(w.apply_silu), stream(dev))
    assert code == gn.GnStatus.OK, gn.status_text(code)
    torch.cuda.synchronize()
    y_bits = from_dev_bits(y)
    del x, y
    ref = oracle.gn_silu(x_bits, gamma, beta, w.N, w.L, w.C, w.G, w.eps, w.apply_silu,
                         out_dtype=np.float32)
    compare(y_bits, ref, "gn_silu_nhwc " + w.name)


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_extra_workload_full_size(gn, dev, oracle, idx):
    """The shapes bench.py measures beside the decoder shapes, full size, through
    the rows entry (the one the rows case uses; NHWC is the same call)."""
    from gn_inputs import EXTRA_WORKLOADS, make_inputs
    w = EXTRA_WORKLOADS[idx]
    print("case %s %s silu=%d" % (w.name, w.label(), w.apply_silu), flush=True)
    x_bits, gamma, beta = make_inputs(w)
    y_bits = run_rows(gn, dev, x_bits, gamma, beta, w.N, w.L, w.C, w.G, w.eps, w.apply_silu)
    ref = oracle.gn_silu(x_bits, gamma, beta, w.N, w.L, w.C, w.G, w.eps, w.apply_silu,
                         out_dtype=np.float32)
    compare(y_bits, ref, w.name)


def test_beyond_2_31_elements_periodic(gn, dev, oracle):
    """A sample of more than 2^31 elements (4 GiB of bf16): 64-bit offsets in
    both steps.  x repeats a P-row block R times along the rows, so the exact
    group statistics over all L = R*P rows are those of one block and every
    output row l equals the oracle's output row l mod P; rows of the first
    block, rows around element 2^31 and the last rows are compared."""
    from gn_inputs import make_custom
    P, C, G, R = 4096, 512, 32, 1025
    L = P * R
    assert L * C > 2 ** 31
    blk_bits, gamma, beta = make_custom(1, P, C, seed=77, mean_range=(-1, 1), std_range=(0.5, 2))
    ref = oracle.gn_silu(blk_bits, gamma, beta, 1, P, C, G, 1e-6, 1).reshape(P, C)
    print("case periodic N=1 L=%d C=%d G=%d (%d elements)" % (L, C, G, L * C), flush=True)
    blk = to_dev_bits(blk_bits, dev).reshape(P, C)
    x = blk.repeat(R, 1).reshape(1, L, C)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    with torch.no_grad():
        y = gn.group_norm_silu_rows(x, G, g, b, 1e-6)
    torch.cuda.synchronize()
    del x
    mid = 2 ** 31 // C
    rows = np.concatenate([np.arange(0, P), np.arange(mid - 8, mid + 8), np.arange(L - 300, L)])
    got = from_dev_bits(y[0, torch.from_numpy(rows).to(dev)])
    compare(got, ref[rows % P], "periodic beyond 2^31")


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_decoder_workload_statistics(gn, dev, oracle, idx):
    """fp32 mean/rstd against the oracle's fp64 ones.

    Bounds: the sums are of pivot-shifted values in runs of at most a few
    hundred per lane plus fixed trees, so S/M and Q/M carry relative error of
    order 1e-6; hence |dmean| <= 1e-4*std + 2^-22*|mean| and |drstd|/rstd <= 1e-4.
    """
    from gn_inputs import WORKLOADS, make_inputs
    w = WORKLOADS[idx]
    x_bits, _, _ = make_inputs(w)
    x = to_dev_bits(x_bits, dev).reshape(w.N, w.L, w.C)
    with torch.no_grad():
        mean, rstd = gn.group_stats_rows(x, w.G, w.eps)
    torch.cuda.synchronize()
    m_ref, v_ref = oracle.group_stats(x_bits, w.N, w.L, w.C, w.G)
    r_ref = 1.0 / np.sqrt(v_ref + np.float64(np.float32(w.eps)))
    m = mean.cpu().numpy().astype(np.float64)
    r = rstd.cpu().numpy().astype(np.float64)
    dm = np.abs(m - m_ref)
    assert np.all(dm <= 1e-4 * np.sqrt(v_ref) + 2.0 ** -22 * np.abs(m_ref)), dm.max()
    dr = np.abs(r - r_ref) / r_ref
    print("%s stats: max|dmean|=%.2e max rel drstd=%.2e" % (w.name, dm.max(), dr.max()))
    assert np.all(dr <= 1e-4), dr.max()


# --------------------------------------------------------------- edge cases
SWEEP = []
for _C in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048):
    for _G in sorted({1, min(32, _C), _C}):
        for _N, _L in ((1, 1), (2, 3), (1, 257), (2, 1000)):
            SWEEP.append((_N, _L, _C, _G))


@pytest.mark.parametrize("N,L,C,G", SWEEP)
def test_shape_sweep(gn, dev, oracle, N, L, C, G):
    from gn_inputs import make_custom
    x_bits, gamma, beta = make_custom(N, L, C, seed=N * 7919 + L * 31 + C * 3 + G,
                                      mean_range=(-3, 3), std_range=(0.3, 2))
    for silu in (0, 1):
        y = run_rows(gn, dev, x_bits, gamma, beta, N, L, C, G, 1e-6, silu)
        ref = oracle.gn_silu(x_bits, gamma, beta, N, L, C, G, 1e-6, silu)
        compare(y, ref, "sweep N=%d L=%d C=%d G=%d silu=%d" % (N, L, C, G, silu))


@pytest.mark.parametrize("N,L,C,G", [
    (3, 70001, 128, 32),    # several tiles per workgroup, unrolled + remainder + ragged tail
    (2, 5000, 64, 8),       # partial last tile
    (2, 131072, 64, 8),     # many chunks per sample
    (1, 4099, 2048, 2048),  # widest rows, one channel per group
    (1, 4099, 2048, 1),     # widest rows, one group
    (5, 999, 4, 2),         # 2-byte lanes (L*C not a multiple of 8), several samples
])
def test_multi_tile_ragged(gn, dev, oracle, N, L, C, G):
    from gn_inputs import make_custom
    x_bits, gamma, beta = make_custom(N, L, C, seed=L + C + G, mean_range=(-6, 6),
                                      std_range=(0.2, 1.5))
    y = run_rows(gn, dev, x_bits, gamma, beta, N, L, C, G, 1e-6, 1)
    ref = oracle.gn_silu(x_bits, gamma, beta, N, L, C, G, 1e-6, 1)
    compare(y, ref, "ragged N=%d L=%d C=%d G=%d" % (N, L, C, G))


def test_rows_variant_as_attention(gn, dev, oracle):
    """(N, L, C) = (1, 16384, 512), G=32, no SiLU, through group_norm_silu_rows."""
    from gn_inputs import make_custom
    N, L, C, G = 1, 16384, 512, 32
    x_bits, gamma, beta = make_custom(N, L, C, seed=4242, mean_range=(-1, 1), std_range=(0.5, 2))
    x = to_dev_bits(x_bits, dev).reshape(N, L, C)
    with torch.no_grad():
        y = gn.group_norm_silu_rows(x, G, torch.from_numpy(gamma).to(dev),
                                    torch.from_numpy(beta).to(dev), 1e-6, apply_silu=False)
    torch.cuda.synchronize()
    ref = oracle.gn_silu(x_bits, gamma, beta, N, L, C, G, 1e-6, False)
    compare(from_dev_bits(y), ref, "rows attention")


# In place (y == x): step 3 overwrites x while other workgroups of the same
# sample still run, so nothing in step 3 may read x beyond its own elements
# (the late finalize takes its group pivots from step 1, not from x).  Late
# finalize shapes (x <= 16 MiB) and a fused one.
@pytest.mark.parametrize("N,L,C,G", [(2, 3000, 256, 32), (1, 16384, 512, 32), (8, 512, 128, 32),
                                     (3, 777, 320, 32), (1, 65536, 512, 32)])
def test_in_place(gn, dev, oracle, N, L, C, G):
    from gn_inputs import make_custom
    x_bits, gamma, beta = make_custom(N, L, C, seed=11, mean_range=(-2, 2))
    y = run_rows(gn, dev, x_bits, gamma, beta, N, L, C, G, 1e-6, 1, inplace=True)
    y_oop = run_rows(gn, dev, x_bits, gamma, beta, N, L, C, G, 1e-6, 1)
    assert np.array_equal(y, y_oop), "in place differs from out of place"
    compare(y, oracle.gn_silu(x_bits, gamma, beta, N, L, C, G, 1e-6, 1), "in place")


def test_no_affine(gn, dev, oracle):
    from gn_inputs import make_custom
    N, L, C, G = 2, 777, 64, 16
    x_bits, _, _ = make_custom(N, L, C, seed=12, mean_range=(-2, 2))
    for silu in (0, 1):
        y = run_rows(gn, dev, x_bits, None, None, N, L, C, G, 1e-6, silu)
        compare(y, oracle.gn_silu(x_bits, None, None, N, L, C, G, 1e-6, silu), "no affine")


def test_large_eps_and_constant_groups(gn, dev, oracle):
    from gn_inputs import f32_to_bf16_bits
    N, L, C, G = 1, 4096, 64, 8
    xf = np.random.default_rng(5).normal(0, 1, (N, L, C)).astype(np.float32)
    xf[:, :, :8] = 2.5  # group 0 constant: output = beta (then SiLU)
    x_bits = f32_to_bf16_bits(xf).reshape(-1)
    gamma = np.linspace(0.5, 1.5, C).astype(np.float32)
    beta = np.linspace(-1, 1, C).astype(np.float32)
    for eps in (1e-6, 0.5):
        y = run_rows(gn, dev, x_bits, gamma, beta, N, L, C, G, eps, 1)
        compare(y, oracle.gn_silu(x_bits, gamma, beta, N, L, C, G, eps, 1), "eps=%g" % eps)


def test_exact_statistics_integer_inputs(gn, dev):
    """Integer x in [-2, 2] with M = L*Cg a power of two and sum of squares
    below 2^24: every fp32 sum is exact in any order, so the mean must be the
    exact mean and rstd the correctly rounded 1/sqrt(var + eps).  Catches a
    dropped or doubled tile, chunk or workgroup.
    """
    from gn_inputs import f32_to_bf16_bits
    N, L, C, G = 2, 131072, 64, 8           # M = 2^20 per group, 1024 chunks per sample
    xi = np.random.default_rng(21).integers(-2, 3, N * L * C).astype(np.float32)
    x_bits = f32_to_bf16_bits(xi)
    x = to_dev_bits(x_bits, dev).reshape(N, L, C)
    eps = 1e-6
    with torch.no_grad():
        mean, rstd = gn.group_stats_rows(x, G, eps)
    torch.cuda.synchronize()
    xs = xi.reshape(N, L, G, C // G).astype(np.int64)
    M = L * (C // G)
    S = xs.sum(axis=(1, 3))
    Q = (xs * xs).sum(axis=(1, 3))
    exact_mean = S / M                       # exact in fp64 (M is a power of two)
    exact_var = Q / M - exact_mean ** 2      # exact dyadic rationals
    want_r = (1.0 / np.sqrt(exact_var + np.float64(np.float32(eps)))).astype(np.float32)
    assert np.array_equal(mean.cpu().numpy(), exact_mean.astype(np.float32))
    got_r = rstd.cpu().numpy()
    ulp = np.abs(got_r.view(np.int32) - want_r.view(np.int32))
    assert ulp.max() <= 1, ulp.max()


# (N, L, C, G, dtype): shapes whose full path runs the late finalize (step 2
# inside every step-3 workgroup; the 16 MiB decoder shape among them), the
# separate finalize kernel ((1, 65536, 512): 64 MiB; G = 512) or the fused
# tail of step 1 ((1, 163848, 512): 160 MiB + 8 KiB).  gn_stats_rows runs the fused tail where the full path runs
# the late finalize (the same order of additions), else the full path's own
# step 2.
SPLIT_CASES = [
    (2, 20000, 128, 32, "bf16"), (1, 16384, 512, 32, "bf16"), (1, 4096, 128, 32, "bf16"),
    (3, 777, 320, 32, "bf16"), (2, 1000, 64, 1, "bf16"), (1, 3000, 256, 256, "bf16"),
    (4, 4096, 512, 32, "bf16"), (1, 16384, 512, 32, "f16"), (1, 8192, 256, 32, "f32"),
    (2, 9, 8, 8, "bf16"), (1, 300, 256, 256, "bf16"), (1, 65536, 512, 32, "bf16"),
    (1, 2000, 512, 512, "bf16"), (1, 163848, 512, 32, "bf16"),
]


@pytest.mark.parametrize("N,L,C,G,dt", SPLIT_CASES)
def test_stats_then_apply_equals_full_path(gn, dev, N, L, C, G, dt):
    """The full path equals steps 1-2 (gn_stats_rows) followed by step 3 given
    mean/rstd, bit for bit, whichever finalize the full path runs."""
    from gn_inputs import make_custom
    x_np, gamma, beta = make_custom(N, L, C, seed=31, mean_range=(-2, 2), dtype=dt)
    if dt == "bf16":
        x = to_dev_bits(x_np, dev).reshape(N, L, C)
    else:
        x = torch.from_numpy(x_np).to(dev).reshape(N, L, C)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    late = gn.plan_rows(N, L, C, G, gn.dtype_code(x.dtype))["late_finalize"]
    print("case N=%d L=%d C=%d G=%d %s late=%d" % (N, L, C, G, dt, late), flush=True)
    with torch.no_grad():
        full = gn.group_norm_silu_rows(x, G, g, b, 1e-6)
        mean, rstd = gn.group_stats_rows(x, G, 1e-6)
        split = gn.apply_rows(x, mean, rstd, g, b, apply_silu=True)
    torch.cuda.synchronize()
    iv = torch.int32 if dt == "f32" else torch.int16
    assert torch.equal(full.view(iv), split.view(iv))


def test_deterministic_repeats(gn, dev):
    from gn_inputs import WORKLOADS, make_inputs
    w = WORKLOADS[1]
    x_bits, gamma, beta = make_inputs(w)
    x = to_dev_bits(x_bits, dev).reshape(w.N, w.L, w.C)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    outs = []
    with torch.no_grad():
        for _ in range(5):
            outs.append(gn.group_norm_silu_rows(x, w.G, g, b, w.eps).view(torch.int16).clone())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_canaries_around_output(gn, dev, oracle):
    """Writes stay inside y: guard regions on both sides keep their bytes."""
    from gn_inputs import make_custom
    N, L, C, G = 1, 5000, 128, 32
    x_bits, gamma, beta = make_custom(N, L, C, seed=77)
    n = N * L * C
    pad = 4096
    buf = torch.full((n + 2 * pad,), 0x5A5A, dtype=torch.int16, device=dev)
    y = buf[pad:pad + n]
    x = to_dev_bits(x_bits, dev)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    code = gn.gn_silu_rows(vp(x), vp(g), vp(b), vp(y), N, L, C, G, 1e-6, 1, stream(dev))
    assert code == 0
    torch.cuda.synchronize()
    assert bool((buf[:pad] == 0x5A5A).all()) and bool((buf[pad + n:] == 0x5A5A).all())
    compare(from_dev_bits(y), oracle.gn_silu(x_bits, gamma, beta, N, L, C, G, 1e-6, 1), "canary")


def test_side_stream(gn, dev, oracle):
    from gn_inputs import make_custom
    N, L, C, G = 1, 9000, 256, 32
    x_bits, gamma, beta = make_custom(N, L, C, seed=91)
    s = torch.cuda.Stream(dev)
    x = to_dev_bits(x_bits, dev).reshape(N, L, C)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s), torch.no_grad():
        y = gn.group_norm_silu_rows(x, G, g, b, 1e-6)
    s.synchronize()
    compare(from_dev_bits(y), oracle.gn_silu(x_bits, gamma, beta, N, L, C, G, 1e-6, 1), "stream")


def test_profile_helper(gn, dev):
    from gn_inputs import WORKLOADS, make_inputs
    w = WORKLOADS[2]
    x_bits, gamma, beta = make_inputs(w)
    x = to_dev_bits(x_bits, dev).reshape(w.N, w.L, w.C)
    y = torch.empty_like(x)
    ms = gn.profile_rows(x, w.G, torch.from_numpy(gamma).to(dev), torch.from_numpy(beta).to(dev),
                         w.eps, True, y, 3)
    # G = 32, large: the statistics kernel finishes the groups itself (no finalize launch)
    assert set(ms) == {"gn_partial_stats", "gn_apply"}
    assert all(v > 0 for v in ms.values())
    x2 = to_dev_bits(make_inputs(w)[0][: 8 * 16384 * 512], dev).reshape(8, 16384, 512)
    assert not gn.plan_single_launch(8, 16384, 512, 512)["single_launch"]
    ms2 = gn.profile_rows(x2, 512, None, None, w.eps, True, torch.empty_like(x2), 2)
    # G = 512 > 256 threads: a separate finalize kernel
    assert set(ms2) == {"gn_partial_stats", "gn_finalize_stats", "gn_apply"}
    # a small tensor: the single launch, nothing else
    x3 = x2[:2, :1024, :256].contiguous()
    assert gn.plan_single_launch(2, 1024, 256, 32)["single_launch"]
    ms3 = gn.profile_rows(x3, 32, None, None, w.eps, True, torch.empty_like(x3), 2)
    assert set(ms3) == {"gn_strip"} and ms3["gn_strip"] > 0


# ------------------------------------------------------ unsupported contract
def test_unsupported_inputs_return_none(gn, dev):
    x = torch.randn(1, 64, 8, 8, device=dev).to(torch.bfloat16)  # NCHW-contiguous
    g = torch.ones(64, device=dev)
    with torch.no_grad():
        assert gn.group_norm_silu_4d(x, 32, g, g) is None                          # not channels_last
        xc = x.to(memory_format=torch.channels_last)
        assert gn.group_norm_silu_4d(xc, 32, g, g) is not None
        assert gn.group_norm_silu_4d(xc.half(), 32, g.half(), g.half()) is not None  # fp16
        assert gn.group_norm_silu_4d(xc, 32, g.double(), g.double()) is None       # fp64 affine
        assert gn.group_norm_silu_4d(xc, 32, g.half(), g) is None                  # mixed affine
        assert gn.group_norm_silu_4d(xc.double(), 32, g, g) is None                # fp64 x
        x3k = torch.randn(1, 3000, 4, 4, device=dev).to(torch.bfloat16).to(memory_format=torch.channels_last)
        assert gn.group_norm_silu_4d(x3k, 8) is None                               # no tile layout
        x16k = torch.randn(1, 16384, 2, 2, device=dev).to(torch.bfloat16).to(memory_format=torch.channels_last)
        assert gn.group_norm_silu_4d(x16k, 32) is None                             # C > 8192
        assert gn.group_norm_silu_4d(xc, 32, g.cpu(), g.cpu()) is None             # host affine
        with pytest.raises(ValueError):
            gn.group_norm_silu_4d(xc, 7)                                           # C % G != 0
    assert gn.group_norm_silu_4d(xc, 32, g, g) is None                             # grad enabled


def test_host_pointer_is_unsupported(gn, dev):
    host = np.zeros(1024, np.uint16)
    y = torch.empty(1024, dtype=torch.int16, device=dev)
    code = gn.gn_silu_rows(ctypes.c_void_p(host.ctypes.data), None, None, vp(y), 1, 16, 64, 32,
                           1e-6, 1, stream(dev))
    assert code == gn.GnStatus.UNSUPPORTED


def test_extent_one_dims_accept_any_stride(gn, dev, oracle):
    from gn_inputs import make_custom
    N, C, H, W, G = 1, 64, 1, 50, 8
    x_bits, gamma, beta = make_custom(N, H * W, C, seed=8)
    x = to_dev_bits(x_bits, dev)
    y = torch.empty_like(x)
    st_x = (ctypes.c_int64 * 4)(12345, 1, 999, C)  # N and H have extent 1
    st_y = (ctypes.c_int64 * 4)(7, 1, 3, C)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    code = gn.gn_silu_nhwc_strided(vp(x), st_x, vp(g), vp(b), vp(y), st_y, N, H, W, C, G, 1e-6, 1,
                                   stream(dev))
    assert code == 0
    torch.cuda.synchronize()
    compare(from_dev_bits(y), oracle.gn_silu(x_bits, gamma, beta, N, H * W, C, G, 1e-6, 1),
            "extent-1 strides")


def test_sample_count_changes_on_one_stream(gn, dev, oracle):
    """The per-sample arrival counters live at the front of the stream's
    scratch and only grow; calls whose N rises and falls on the same stream
    must each see cleared counters (a stale counter would skip or repeat the
    finalize of a sample)."""
    from gn_inputs import make_custom
    L, C, G = 3000, 64, 16
    for N in (1, 9, 3, 40, 2, 40, 1):
        x_bits, gamma, beta = make_custom(N, L, C, seed=100 + N, mean_range=(-2, 2))
        for rep in range(2):
            y = run_rows(gn, dev, x_bits, gamma, beta, N, L, C, G, 1e-6, 1)
            compare(y, oracle.gn_silu(x_bits, gamma, beta, N, L, C, G, 1e-6, 1),
                    "N=%d rep %d" % (N, rep))


def test_many_samples_one_workgroup_each(gn, dev, oracle):
    """N above the statistics workgroup target: one workgroup per sample, each
    of which is also the last to arrive for its sample."""
    from gn_inputs import make_custom
    N, L, C, G = 300, 64, 32, 8
    x_bits, gamma, beta = make_custom(N, L, C, seed=300, mean_range=(-3, 3))
    assert gn.plan_rows(N, L, C, G)["K1"] == 1
    y = run_rows(gn, dev, x_bits, gamma, beta, N, L, C, G, 1e-6, 1)
    compare(y, oracle.gn_silu(x_bits, gamma, beta, N, L, C, G, 1e-6, 1), "N=300")


def test_device_info_reports_the_device(gn, dev):
    info = gn.device_info(dev.index or 0)
    props = torch.cuda.get_device_properties(dev)
    assert info["compute_units"] == props.multi_processor_count
    assert info["wavefront"] == 64
    assert info["memory_bytes"] == props.total_memory
    assert info["engine_clock_khz"] > 0 and info["memory_clock_khz"] > 0
    assert info["memory_bus_bits"] > 0


def test_arrival_counters_alternating_modes(gn, dev, oracle):
    """Shapes whose samples have >= 64 statistics chunks (two-level arrival
    count) alternate on one stream with shapes that use one counter word per
    sample: every repeat is bitwise equal to the first call of its shape (a
    counter left non-zero would misplace the finalize), and the two-level one
    matches the oracle."""
    from gn_inputs import make_custom
    # (above 160 MiB the statistics kernel finishes the groups itself: the
    # arrival counts run there)
    cases = [(3, 250001, 128, 32), (1, 4096, 128, 32), (2, 200000, 256, 32), (16, 16384, 512, 32)]
    ks = [gn.plan_rows(*c)["K1"] for c in cases]
    assert ks[0] >= 64 and ks[2] >= 64 and ks[1] < 64 and ks[3] < 64
    data = []
    for i, (N, L, C, G) in enumerate(cases):
        x_bits, gamma, beta = make_custom(N, L, C, seed=300 + i)
        data.append((to_dev_bits(x_bits, dev).reshape(N, L, C), torch.from_numpy(gamma).to(dev),
                     torch.from_numpy(beta).to(dev), x_bits, gamma, beta))
    first = {}
    with torch.no_grad():
        for rep in range(3):
            for i, (N, L, C, G) in enumerate(cases):
                x, g, b = data[i][:3]
                y = gn.group_norm_silu_rows(x, G, g, b, 1e-6).view(torch.int16).clone()
                if rep == 0:
                    first[i] = y
                else:
                    assert torch.equal(y, first[i]), (rep, cases[i])
    torch.cuda.synchronize()
    N, L, C, G = cases[0]
    x_bits, gamma, beta = data[0][3:]
    compare(from_dev_bits(first[0].view(torch.bfloat16)),
            oracle.gn_silu(x_bits, gamma, beta, N, L, C, G, 1e-6, 1), "two-level arrival")


# ------------------------------------------------------------- HIP graphs
def test_graph_replays_after_the_scratch_grows(gn, dev):
    """A GroupNorm captured into a HIP graph keeps the stream's scratch buffer
    of capture time.  A later call on the same stream that needs a larger
    buffer retires the old one without freeing it, so every replay, before
    and after, equals the eager result bit for bit."""
    small, big = (1, 4096, 128, 32), (4, 16384, 512, 32)
    assert gn.plan_rows(*small)["scratch_bytes"] <= 1 << 16 < gn.plan_rows(*big)["scratch_bytes"]
    gen = torch.Generator(device="cpu").manual_seed(21)
    xs = torch.randn(small[:3], generator=gen).bfloat16().to(dev)
    xb = torch.randn(big[:3], generator=gen).bfloat16().to(dev)
    stream = torch.cuda.Stream(dev)
    with torch.no_grad():
        with torch.cuda.stream(stream):
            ref = gn.group_norm_silu_rows(xs, 32).clone()  # allocates the stream's scratch
            gn.group_norm_silu_rows(xs, 32)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            out = gn.group_norm_silu_rows(xs, 32)
        for rep in range(3):
            with torch.cuda.stream(stream):
                g.replay()
                refb = gn.group_norm_silu_rows(xb, 32)  # grows the scratch on the first pass
            stream.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "replay %d" % rep
            with torch.cuda.stream(stream):
                g.replay()                               # after the growth
                again = gn.group_norm_silu_rows(xb, 32)
            stream.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "replay %d" % rep
            assert torch.equal(again.view(torch.int16), refb.view(torch.int16))


def test_counters_recover_after_overlapping_calls(gn, dev):
    """A graph captured on stream A and replayed on stream B while eager calls
    run on A: the overlapping calls share A's scratch (the header calls their
    results undefined; no kernel waits on another, so they all finish).
    Afterwards every call on A is bitwise the reference again: step 3 clears
    the arrival counters step 1 used, so nothing the overlap left behind
    reaches the later calls."""
    N, L, C, G = 1, 196608, 512, 32       # 192 MiB, 256 chunks: the two-level arrival count
    p = gn.plan_rows(N, L, C, G)
    assert p["K1"] >= 64 and not p["late_finalize"]
    assert not gn.plan_single_launch(N, L, C, G)["single_launch"]
    gen = torch.Generator(device="cpu").manual_seed(77)
    x = torch.randn(N, L, C, generator=gen).bfloat16().to(dev)
    a, b = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    with torch.no_grad():
        with torch.cuda.stream(a):
            ref = gn.group_norm_silu_rows(x, G).clone()
            gn.group_norm_silu_rows(x, G)
        a.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=a):
            gn.group_norm_silu_rows(x, G)
        for _ in range(20):                   # overlap: B replays while A computes
            with torch.cuda.stream(b):
                g.replay()
            with torch.cuda.stream(a):
                gn.group_norm_silu_rows(x, G)
        torch.cuda.synchronize()
        for rep in range(5):
            with torch.cuda.stream(a):
                y = gn.group_norm_silu_rows(x, G)
            a.synchronize()
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), "call %d after" % rep

"""GPU parity for fp16 and fp32 input/output, against the fp64 oracle.

The page's kernel tests cover fp32 as well as bf16 activations ("FLUX.2 VAE
decoder fast path behind quality=high", Accuracy section, unit tests); the
library computes in fp32 for every element type and rounds y once to it.
Tolerances, per element (NaN never passes), derived from the arithmetic:

  fp16:  |y - ref| <= 1e-4 + 1e-3*|ref|   (rounding to fp16 <= 2^-11 relative;
         fp32 statistics and the shifted fma add < 1e-5 relative and a few
         1e-6 absolute)
  fp32:  |y - ref| <= 2e-4 + 2e-4*|ref|   (no output rounding to speak of;
         the fp32 sums of up to 1024 terms per lane bound the relative error
         of the variance by ~6e-5 in the worst case, so z is off by <= 3e-5
         relative, plus the shifted fma and the SiLU's exp2/rcp)
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = {"f16": (1e-4, 1e-3), "f32": (2e-4, 2e-4)}
TORCH = {"f16": torch.float16, "f32": torch.float32}
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
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def to_host(t):
    return t.contiguous().cpu().numpy().reshape(-1)


def compare(y, ref, dtype, what):
    atol, rtol = TOL[dtype]
    ref = ref.reshape(-1).astype(np.float64)
    got = y.astype(np.float64)
    err = np.abs(got - ref)
    ok = err <= atol + rtol * np.abs(ref)
    bad = int(np.count_nonzero(~ok))
    first = None
    if bad:
        i = int(np.flatnonzero(~ok)[0])
        first = (i, float(got[i]), float(ref[i]))
    worst = float(np.nanmax(err)) if err.size else 0.0
    rel = float(np.nanmax(err / (atol + rtol * np.abs(ref)))) if err.size else 0.0
    print("%s: max|y-ref|=%.3e max err/tol=%.3f violations=%d/%d first=%s"
          % (what, worst, rel, bad, ref.size, first), flush=True)
    assert bad == 0, "%s: %d elements outside tolerance, first %s" % (what, bad, first)


def vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("idx", [0, 1, 4])
def test_decoder_workloads(gn, dev, oracle, dtype, idx):
    from gn_inputs import WORKLOADS, make_inputs
    w = WORKLOADS[idx]
    print("case %s %s %s" % (w.name, w.label(), dtype), flush=True)
    x, gamma, beta = make_inputs(w, dtype=dtype)
    xt = to_dev(x, dev).reshape(w.N, w.H, w.W, w.C).permute(0, 3, 1, 2)
    assert xt.dtype == TORCH[dtype]
    with torch.no_grad():
        y = gn.group_norm_silu_4d(xt, w.G, to_dev(gamma, dev), to_dev(beta, dev), w.eps)
    assert y is not None and y.dtype == TORCH[dtype]
    torch.cuda.synchronize()
    got = to_host(y.permute(0, 2, 3, 1))
    ref = oracle.gn_silu(x, gamma, beta, w.N, w.L, w.C, w.G, w.eps, True, out_dtype=np.float32)
    compare(got, ref, dtype, "%s %s" % (w.name, dtype))


def test_largest_workload_fp32(gn, dev, oracle):
    """(1,256,1024,1024) in fp32: 1 GiB per tensor, so step 3 streams x with
    nontemporal loads (the cache-residency threshold counts bytes)."""
    from gn_inputs import WORKLOADS, make_inputs
    w = WORKLOADS[3]
    assert gn.plan_rows(w.N, w.L, w.C, w.G, gn.GnDtype.F32)["apply_nontemporal_loads"] == 1
    x, gamma, beta = make_inputs(w, dtype="f32")
    xt = to_dev(x, dev).reshape(w.N, w.L, w.C)
    with torch.no_grad():
        y = gn.group_norm_silu_rows(xt, w.G, to_dev(gamma, dev), to_dev(beta, dev), w.eps)
    torch.cuda.synchronize()
    got = to_host(y)
    del xt, y
    ref = oracle.gn_silu(x, gamma, beta, w.N, w.L, w.C, w.G, w.eps, True, out_dtype=np.float32)
    compare(got, ref, "f32", "%s f32" % w.name)


SWEEP = [(N, L, C, G) for C in (1, 4, 8, 64, 512, 2048) for G in sorted({1, min(32, C), C})
         for (N, L) in ((1, 3), (2, 1001))]


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("N,L,C,G", SWEEP)
def test_shape_sweep(gn, dev, oracle, dtype, N, L, C, G):
    from gn_inputs import make_custom
    x, gamma, beta = make_custom(N, L, C, seed=N * 31 + L + C * 7 + G, mean_range=(-3, 3),
                                 std_range=(0.3, 2), dtype=dtype)
    xt = to_dev(x, dev).reshape(N, L, C)
    g, b = to_dev(gamma, dev), to_dev(beta, dev)
    for silu in (False, True):
        with torch.no_grad():
            y = gn.group_norm_silu_rows(xt, G, g, b, 1e-6, apply_silu=silu)
        torch.cuda.synchronize()
        compare(to_host(y), oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, silu), dtype,
                "sweep %s N=%d L=%d C=%d G=%d silu=%d" % (dtype, N, L, C, G, silu))


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_in_place_and_repeatable(gn, dev, oracle, dtype):
    from gn_inputs import make_custom
    N, L, C, G = 2, 40000, 128, 32
    x, gamma, beta = make_custom(N, L, C, seed=8, mean_range=(-5, 5), std_range=(0.2, 1),
                                 dtype=dtype)
    g, b = to_dev(gamma, dev), to_dev(beta, dev)
    xt = to_dev(x, dev).reshape(N, L, C)
    with torch.no_grad():
        a = gn.group_norm_silu_rows(xt, G, g, b, 1e-6)
        a2 = gn.group_norm_silu_rows(xt, G, g, b, 1e-6)
        mean, rstd = gn.group_stats_rows(xt, G, 1e-6)
        split = gn.apply_rows(xt, mean, rstd, g, b, apply_silu=True)
        y = gn.group_norm_silu_rows(xt, G, g, b, 1e-6, out=xt)  # in place
    torch.cuda.synchronize()
    assert y.data_ptr() == xt.data_ptr()
    assert torch.equal(a, a2) and torch.equal(a, split) and torch.equal(a, xt)
    compare(to_host(a), oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, True), dtype,
            "in place %s" % dtype)


def test_statistics_fp32(gn, dev, oracle):
    from gn_inputs import WORKLOADS, make_inputs
    w = WORKLOADS[4]
    x, _, _ = make_inputs(w, dtype="f32")
    xt = to_dev(x, dev).reshape(w.N, w.L, w.C)
    with torch.no_grad():
        mean, rstd = gn.group_stats_rows(xt, w.G, w.eps)
    torch.cuda.synchronize()
    m_ref, v_ref = oracle.group_stats(x, w.N, w.L, w.C, w.G)
    r_ref = 1.0 / np.sqrt(v_ref + np.float64(np.float32(w.eps)))
    dm = np.abs(mean.cpu().numpy() - m_ref)
    dr = np.abs(rstd.cpu().numpy() - r_ref) / r_ref
    print("fp32 stats: max|dmean|=%.2e max rel drstd=%.2e" % (dm.max(), dr.max()))
    assert np.all(dm <= 1e-4 * np.sqrt(v_ref) + 2.0 ** -22 * np.abs(m_ref))
    assert np.all(dr <= 1e-4)


def test_other_dtypes_declined(gn, dev):
    x = torch.randn(1, 64, 4, 4, device=dev, dtype=torch.float64).to(memory_format=torch.channels_last)
    with torch.no_grad():
        assert gn.group_norm_silu_4d(x, 32) is None
        assert gn.group_norm_silu_4d(x.to(torch.int32), 32) is None

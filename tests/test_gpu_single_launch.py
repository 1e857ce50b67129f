"""GPU parity of the single launch (gn_strip): steps 1-3 in one kernel, one
workgroup per strip of whole groups, for the small tensors whose plan takes
it (gn_plan_single_launch).

Every case first asserts that its shape takes the single launch, then
compares with the fp64 oracle element by element at the tolerances of the
other parity tests (bf16 1e-2 + 1.6e-2|ref|, fp16 1e-4 + 1e-3|ref|, fp32
2e-4 + 2e-4|ref|; NaN never passes), and checks the properties the path
promises: in place equals out of place bit for bit, steps 1-2 then 3 (which
take the single launch's statistics) equal the full path bit for bit,
repeated calls are bitwise identical, the no-allocation entry gives the same
bits.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-2, 1.6e-2), "f16": (1e-4, 1e-3), "f32": (2e-4, 2e-4)}
CODE = {"bf16": 0, "f16": 1, "f32": 2}

# (N, L, C, G): every piece / group split the kernel has -- Cg = 1, 2, 4
# (several groups per 16-byte piece), Cg = 8 (one piece), Cg = 16 ... 512
# (2 ... 64 pieces per group) -- ragged row counts, one and two pieces per
# lane, 1 to 256 workgroups, XCD order on and off.
SHAPES = [
    (2, 1024, 256, 32), (8, 1024, 128, 32), (1, 2048, 128, 32), (4, 2048, 256, 32),
    (3, 999, 64, 32), (2, 77, 8, 8), (1, 5, 16, 1), (4, 1000, 128, 128), (2, 513, 256, 256),
    (1, 1, 8, 1), (5, 123, 16, 16), (1, 1024, 32, 32), (2, 256, 1024, 32), (1, 32, 4096, 8),
    (1, 16, 2048, 4), (2, 1000, 512, 32), (16, 1024, 128, 32), (16, 256, 64, 32),
    (1, 300, 384, 48), (7, 111, 48, 6),
]


@pytest.fixture(scope="module")
def gn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import groupnorm_silu_normalization_amd as g
    return g


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def to_dev(x, dtype, dev):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(dev)


def to_f64(t):
    if t.dtype == torch.bfloat16:
        from gn_inputs import bf16_bits_to_f32
        return bf16_bits_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                                .reshape(-1)).astype(np.float64)
    return t.contiguous().cpu().numpy().reshape(-1).astype(np.float64)


def bits(t):
    return t.contiguous().view(-1).view(torch.uint8).cpu()


def compare(got, ref, dtype, what):
    atol, rtol = TOL[dtype]
    ref = ref.reshape(-1).astype(np.float64)
    err = np.abs(got - ref)
    ok = err <= atol + rtol * np.abs(ref)
    bad = int(np.count_nonzero(~ok))
    first = None
    if bad:
        i = int(np.flatnonzero(~ok)[0])
        first = (i, float(got[i]), float(ref[i]))
    print("%s: max|y-ref|=%.3e violations=%d/%d first=%s" % (
        what, float(np.nanmax(err)) if err.size else 0.0, bad, ref.size, first), flush=True)
    assert bad == 0, "%s: %d elements outside tolerance, first %s" % (what, bad, first)


def run(gn, dev, x, gamma, beta, N, L, C, G, silu, dtype, y=None, eps=1e-6, entry=None):
    y = torch.empty_like(x) if y is None else y
    f = entry or gn.gn_silu_rows_dtype
    code = f(vp(x), vp(gamma), vp(beta), vp(y), N, L, C, G, float(eps), int(silu), CODE[dtype],
             stream(dev))
    assert code == gn.GnStatus.OK, gn.status_text(code)
    return y


def single(gn, N, L, C, G, dtype):
    q = gn.plan_single_launch(N, L, C, G, CODE[dtype])
    assert q["single_launch"] == 1, ("shape does not take the single launch", N, L, C, G, dtype)
    return q


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("N,L,C,G", SHAPES)
def test_single_launch_against_the_oracle(gn, dev, oracle, N, L, C, G, dtype):
    if dtype == "f32" and gn.plan_single_launch(N, L, C, G, CODE[dtype])["single_launch"] == 0:
        pytest.skip("fp32 doubles the bytes per row: the three-step path takes this shape")
    q = single(gn, N, L, C, G, dtype)
    print("case single launch N=%d L=%d C=%d G=%d %s %s" % (N, L, C, G, dtype, q), flush=True)
    from gn_inputs import make_custom
    x, gamma, beta = make_custom(N, L, C, seed=N * 7 + L + C, mean_range=(-1, 1),
                                 std_range=(0.5, 2.0), dtype=dtype)
    xd = to_dev(x, dtype, dev).reshape(N, L, C)
    g, b = torch.from_numpy(gamma).to(dev), torch.from_numpy(beta).to(dev)
    for silu in (1, 0):
        y = run(gn, dev, xd, g, b, N, L, C, G, silu, dtype)
        torch.cuda.synchronize()
        ref = oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, silu)
        compare(to_f64(y), ref, dtype, "single launch silu=%d" % silu)


@pytest.mark.parametrize("N,L,C,G", [(2, 1024, 256, 32), (3, 999, 64, 32), (2, 513, 256, 256),
                                     (1, 16, 2048, 4)])
def test_single_launch_variants_bitwise(gn, dev, oracle, N, L, C, G):
    """In place = out of place; stats then apply = the full path; repeats
    identical; the no-allocation entry identical; no affine against the
    oracle; 16-bit gamma/beta holding the fp32 values give the same bits."""
    single(gn, N, L, C, G, "bf16")
    from gn_inputs import make_custom
    x, gamma, beta = make_custom(N, L, C, seed=41 + C, mean_range=(-2, 2), std_range=(0.5, 2.0))
    xd = to_dev(x, "bf16", dev).reshape(N, L, C)
    g, b = torch.from_numpy(gamma).to(dev), torch.from_numpy(beta).to(dev)
    ref = run(gn, dev, xd, g, b, N, L, C, G, 1, "bf16")
    reps = [run(gn, dev, xd, g, b, N, L, C, G, 1, "bf16") for _ in range(3)]
    noalloc = run(gn, dev, xd, g, b, N, L, C, G, 1, "bf16", entry=gn.gn_silu_rows_noalloc)
    inplace = xd.clone()
    run(gn, dev, inplace, g, b, N, L, C, G, 1, "bf16", y=inplace)
    mean = torch.empty(N * G, device=dev)
    rstd = torch.empty(N * G, device=dev)
    assert gn.gn_stats_rows(vp(xd), N, L, C, G, 1e-6, vp(mean), vp(rstd), stream(dev)) == 0
    split = torch.empty_like(xd)
    assert gn.gn_apply_rows(vp(xd), vp(mean), vp(rstd), vp(g), vp(b), vp(split), N, L, C, G, 1,
                            stream(dev)) == 0
    # bf16 gamma/beta: values exactly representable, so the same bits as fp32 ones
    g16, b16 = g.bfloat16(), b.bfloat16()
    y16 = torch.empty_like(xd)
    code = gn.gn_silu_rows_dtype(vp(xd), vp(g16), vp(b16), vp(y16), N, L, C, G, 1e-6, 1,
                                 0 | gn.AFFINE_FLAG[torch.bfloat16], stream(dev))
    assert code == 0
    y32 = run(gn, dev, xd, g16.float(), b16.float(), N, L, C, G, 1, "bf16")
    plain = run(gn, dev, xd, None, None, N, L, C, G, 1, "bf16")
    torch.cuda.synchronize()
    r = bits(ref)
    for t in reps + [noalloc, inplace, split]:
        assert torch.equal(bits(t), r)
    assert torch.equal(bits(y16), bits(y32))
    compare(to_f64(ref), oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, 1), "bf16", "variants")
    compare(to_f64(plain), oracle.gn_silu(x, None, None, N, L, C, G, 1e-6, 1), "bf16", "no affine")
    # the statistics themselves against the oracle's fp64 ones
    m64, v64 = oracle.group_stats(x, N, L, C, G)
    m = mean.cpu().numpy().astype(np.float64)
    rs = rstd.cpu().numpy().astype(np.float64)
    scale = np.sqrt(v64) + 1e-3
    assert np.all(np.abs(m - m64.reshape(-1)) <= 1e-5 * (np.abs(m64.reshape(-1)) + scale.reshape(-1)))
    rref = 1.0 / np.sqrt(v64.reshape(-1) + 1e-6)
    assert np.all(np.abs(rs - rref) <= 2e-5 * rref)


def test_single_launch_cancellation_stress(gn, dev, oracle):
    """Channel means up to +-8 with std 0.25: the pivot shift keeps the fp32
    sums from cancelling."""
    N, L, C, G = 4, 2048, 256, 32
    single(gn, N, L, C, G, "bf16")
    from gn_inputs import make_custom
    x, gamma, beta = make_custom(N, L, C, seed=5, mean_range=(-8, 8), std_range=(0.25, 1.0))
    xd = to_dev(x, "bf16", dev).reshape(N, L, C)
    y = run(gn, dev, xd, torch.from_numpy(gamma).to(dev), torch.from_numpy(beta).to(dev),
            N, L, C, G, 1, "bf16")
    torch.cuda.synchronize()
    compare(to_f64(y), oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, 1), "bf16", "stress")


def test_single_launch_constant_groups_and_profile(gn, dev, oracle):
    """A constant group has variance 0 and normalises to beta (then SiLU), as
    the oracle's definition gives; the profile helper reports the one kernel."""
    N, L, C, G = 2, 1024, 256, 32
    single(gn, N, L, C, G, "bf16")
    from gn_inputs import f32_to_bf16_bits
    xf = np.random.default_rng(9).normal(0, 1, (N, L, C)).astype(np.float32)
    xf[:, :, :8] = 3.0                   # group 0 of every sample constant
    xf[1, :, 8:16] = -1.5                # and group 1 of sample 1
    x = f32_to_bf16_bits(xf).reshape(-1)
    beta = np.linspace(-2, 2, C).astype(np.float32)
    xd = to_dev(x, "bf16", dev).reshape(N, L, C)
    bd = torch.from_numpy(beta).to(dev)
    y = run(gn, dev, xd, None, bd, N, L, C, G, 1, "bf16")
    torch.cuda.synchronize()
    compare(to_f64(y), oracle.gn_silu(x, None, beta, N, L, C, G, 1e-6, 1), "bf16", "constant")
    ms = gn.profile_rows(xd, G, None, bd, 1e-6, True, torch.empty_like(xd), 3)
    assert set(ms) == {"gn_strip"} and ms["gn_strip"] > 0


@pytest.mark.parametrize("N,L,C,G", [(2, 1024, 256, 32), (4, 1024, 128, 128), (1, 16, 2048, 4),
                                     (8, 512, 64, 32)])
def test_single_launch_exact_statistics(gn, dev, N, L, C, G):
    """Integer x in [-2, 2] with M = L*Cg a power of two and every sum of
    squares below 2^24: each fp32 sum is exact in any order, so the mean is the
    exact mean and rstd the correctly rounded 1/sqrt(var + eps).  A dropped
    or doubled piece, lane, wave or entry shows as a wrong mean."""
    single(gn, N, L, C, G, "bf16")
    from gn_inputs import f32_to_bf16_bits
    M = L * (C // G)
    assert M & (M - 1) == 0 and 4 * M < 2 ** 24
    xi = np.random.default_rng(N + C).integers(-2, 3, (N, L, C)).astype(np.float32)
    x = f32_to_bf16_bits(xi).reshape(-1)
    xd = to_dev(x, "bf16", dev).reshape(N, L, C)
    mean = torch.empty(N * G, device=dev)
    rstd = torch.empty(N * G, device=dev)
    assert gn.gn_stats_rows(vp(xd), N, L, C, G, 1e-6, vp(mean), vp(rstd), stream(dev)) == 0
    torch.cuda.synchronize()
    grp = xi.reshape(N, L, G, C // G).transpose(0, 2, 1, 3).reshape(N * G, -1).astype(np.float64)
    mu = grp.mean(axis=1)
    var = ((grp - mu[:, None]) ** 2).mean(axis=1)
    assert np.array_equal(mean.cpu().numpy(), mu.astype(np.float32))
    assert np.array_equal(rstd.cpu().numpy(), (1.0 / np.sqrt(var + np.float64(np.float32(1e-6))))
                          .astype(np.float32))

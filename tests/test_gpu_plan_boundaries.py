"""GPU parity at the edges of the launch plan's modes.

The plan is a function of the shape alone, and it switches between four ways
of running steps 1-3 at fixed tensor sizes:
  * the single launch of short strips (gn_strip) up to 4 MiB,
  * three steps with the late finalize (step 2 in every step-3 workgroup) up
    to 16 MiB,
  * three kernels, step 2 as gn_finalize_stats, from 16 to 160 MiB (and for
    G > 256 at any size),
  * two kernels, step 2 in the tail of the statistics kernel, above 160 MiB.
Each case takes a shape exactly at a threshold and one just above it, checks
that the kernels the library launched (gn_profile_rows reports which ran) are
those of the expected mode, and compares every output element with the fp64
oracle at the parity tolerances (bf16 1e-2 + 1.6e-2|ref|, fp16 1e-4 +
1e-3|ref|, fp32 2e-4 + 2e-4|ref|; NaN never passes).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-2, 1.6e-2), "f16": (1e-4, 1e-3), "f32": (2e-4, 2e-4)}
ESIZE = {"bf16": 2, "f16": 2, "f32": 4}
MIB = 1 << 20

STRIP = {"gn_strip"}
TWO = {"gn_partial_stats", "gn_apply"}
THREE = {"gn_partial_stats", "gn_finalize_stats", "gn_apply"}

CASES = [  # (N, L, C, G, dtype, mode)
    (8, 1024, 256, 32, "bf16", "strip"),        # 4 MiB exactly
    (8, 1032, 256, 32, "bf16", "late"),         # 4 MiB + 32 KiB
    (1, 16384, 512, 32, "bf16", "late"),        # 16 MiB exactly
    (1, 16392, 512, 32, "bf16", "separate"),    # 16 MiB + 8 KiB
    (2, 8192, 512, 32, "bf16", "late"),         # 16 MiB over two samples
    (2, 8196, 512, 32, "bf16", "separate"),
    (1, 16384, 512, 32, "f16", "late"),
    (1, 16392, 512, 32, "f16", "separate"),
    (1, 8192, 512, 32, "f32", "late"),          # 16 MiB of fp32
    (1, 8200, 512, 32, "f32", "separate"),
    (1, 163840, 512, 32, "bf16", "separate"),   # 160 MiB exactly
    (1, 163848, 512, 32, "bf16", "fused"),      # 160 MiB + 8 KiB
    (1, 81920, 512, 32, "f32", "separate"),     # 160 MiB of fp32
    (1, 81928, 512, 32, "f32", "fused"),
    (1, 81928, 1024, 512, "bf16", "separate"),  # G > 256 above 160 MiB
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


def to_dev(x, dtype, dev):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(dev)


def compare(y, ref, dtype, what):
    from gn_inputs import bf16_bits_to_f32
    atol, rtol = TOL[dtype]
    if dtype == "bf16":
        got_all = y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    else:
        got_all = y.contiguous().cpu().numpy().reshape(-1)
    ref = ref.reshape(-1)
    bad, worst, first = 0, 0.0, None
    step = 1 << 24
    for s in range(0, ref.size, step):
        g = got_all[s:s + step]
        got = (bf16_bits_to_f32(g) if dtype == "bf16" else g).astype(np.float64)
        r = ref[s:s + step].astype(np.float64)
        err = np.abs(got - r)
        ok = err <= atol + rtol * np.abs(r)
        nb = int(np.count_nonzero(~ok))
        if nb and first is None:
            i = int(np.flatnonzero(~ok)[0])
            first = (s + i, float(got[i]), float(r[i]))
        bad += nb
        fin = err[np.isfinite(err)]
        if fin.size:
            worst = max(worst, float(fin.max()))
    print("%s: max|y-ref|=%.3e violations=%d/%d first=%s" % (what, worst, bad, ref.size, first),
          flush=True)
    assert bad == 0, "%s: %d elements outside tolerance, first %s" % (what, bad, first)


def test_cases_straddle_the_thresholds():
    """The shapes sit where the text says: at a threshold or one row or a few
    rows past it (sizes in bytes of x)."""
    sizes = {(N, L, C, dt): N * L * C * ESIZE[dt] for N, L, C, G, dt, mode in CASES}
    for (N, L, C, dt), b in sizes.items():
        assert b in (4 * MIB, 16 * MIB, 160 * MIB) or any(
            0 < b - t <= 64 * 1024 for t in (4 * MIB, 16 * MIB, 160 * MIB)), (N, L, C, dt, b)


@pytest.mark.parametrize("N,L,C,G,dtype,mode", CASES)
def test_mode_boundary_against_the_oracle(gn, dev, oracle, N, L, C, G, dtype, mode):
    print("case N=%d L=%d C=%d G=%d %s %s (%d bytes)" % (N, L, C, G, dtype, mode,
                                                       N * L * C * ESIZE[dtype]), flush=True)
    code = gn.GnDtype.BF16 if dtype == "bf16" else (gn.GnDtype.F16 if dtype == "f16"
                                                     else gn.GnDtype.F32)
    single = gn.plan_single_launch(N, L, C, G, int(code))["single_launch"]
    plan = gn.plan_rows(N, L, C, G, int(code))
    assert single == (1 if mode == "strip" else 0)
    if mode != "strip":
        assert plan["late_finalize"] == (1 if mode == "late" else 0)
    from gn_inputs import make_custom
    x, gamma, beta = make_custom(N, L, C, seed=N * 7 + L + C + G, mean_range=(-1, 1),
                                 std_range=(0.5, 2.0), dtype=dtype)
    xd = to_dev(x, dtype, dev).reshape(N, L, C)
    g, b = torch.from_numpy(gamma).to(dev), torch.from_numpy(beta).to(dev)
    y = torch.empty_like(xd)
    ran = set(gn.profile_rows(xd, G, g, b, 1e-6, True, y, 2))
    want = {"strip": STRIP, "late": TWO, "separate": THREE, "fused": TWO}[mode]
    assert ran == want, ("kernels launched", ran, "expected", want)
    with torch.no_grad():  # the binding declines (None) while autograd records
        y = gn.group_norm_silu_rows(xd, G, g, b, 1e-6)
    assert y is not None
    torch.cuda.synchronize()
    ref = oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, 1, out_dtype=np.float32)
    compare(y, ref, dtype, "%s %s" % (mode, dtype))
    del ref

"""GPU parity of step 3 with eight loads in flight per lane.

Step 3 keeps eight 16-byte loads in flight per lane, instead of four, where x
is at most 160 MiB and every step-3 workgroup's tiles make whole batches of
eight (at least 16 tiles, a multiple of 8, the tiles split evenly), for
layouts with one 16-byte access per lane and tile.  These cases reach those
kernels in each form: power-of-two C with the late finalize (Cg = 2, bf16 and
fp16, one and four samples), power-of-two C reading step 2's mean/rstd
(bf16 and fp16), C that is not a power of two (240 and 192 lanes of a
256-lane workgroup, with and without the late finalize), and 320-lane
workgroups; SiLU on and off, gamma/beta present and absent.  Every output
element is compared with the fp64 oracle at the parity tolerances (bf16
1e-2 + 1.6e-2|ref|, fp16 1e-4 + 1e-3|ref|; NaN never passes).
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

TOL = {"bf16": (1e-2, 1.6e-2), "f16": (1e-4, 1e-3)}
CODE = {"bf16": 0, "f16": 1}
ESIZE = {"bf16": 2, "f16": 2}

CASES = [  # N, L, C, G, dtype, silu, affine
    (1, 131072, 64, 32, "bf16", 1, True),     # late finalize, Cg = 2, 16 MiB
    (1, 32768, 256, 32, "f16", 0, True),      # late finalize, fp16, no SiLU
    (4, 4096, 512, 32, "bf16", 1, False),     # late finalize, four samples, no affine
    (1, 32768, 512, 32, "bf16", 0, True),     # separate finalize, 32 MiB
    (1, 8192, 2048, 32, "f16", 1, True),      # separate finalize, fp16, C = 2048
    (1, 8192, 960, 32, "bf16", 1, True),      # 240 lanes busy, late finalize, 15 MiB
    (1, 16384, 768, 24, "f16", 1, False),     # 192 lanes busy, separate finalize
    (1, 32768, 2560, 32, "bf16", 1, True),    # 320-lane workgroups, 160 MiB
]


def takes_deep_step3(plan, nbytes):
    """The plan's choice, from the values gn_plan_rows_dtype exports: x at
    most 160 MiB, tiles per step-3 workgroup a multiple of 8 and at least 16,
    no uneven split, and one access per lane and tile (slots == W)."""
    rem = plan["tiles"] - plan["tpc2"] * plan["K2"]
    return (nbytes <= 160 << 20 and rem == 0 and plan["tpc2"] >= 16 and plan["tpc2"] % 8 == 0
            and plan["slots"] == plan["W"])


def test_cases_reach_the_deep_step3():
    """Every case takes the deeper step 3, and together they reach the late
    finalize and step 2's own kernel, power-of-two and other C, 256- and
    320-lane workgroups."""
    import groupnorm_silu_normalization_amd as gn
    kinds = set()
    for N, L, C, G, dtype, silu, affine in CASES:
        p = gn.plan_rows(N, L, C, G, CODE[dtype])
        assert p is not None
        assert not gn.plan_single_launch(N, L, C, G, CODE[dtype])["single_launch"]
        assert takes_deep_step3(p, N * L * C * ESIZE[dtype]), (N, L, C, G, dtype)
        kinds.add("late" if p["late_finalize"] else "step 2 kernel")
        kinds.add("pow2" if C & (C - 1) == 0 else "other C")
        kinds.add("320 lanes" if p["threads"] == 320 else "256 lanes")
    assert kinds == {"late", "step 2 kernel", "pow2", "other C", "320 lanes", "256 lanes"}


@pytest.fixture(scope="module")
def gn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import groupnorm_silu_normalization_amd as g
    return g


def vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@pytest.mark.gpu
@pytest.mark.parametrize("N,L,C,G,dtype,silu,affine", CASES)
def test_deep_step3_against_the_oracle(gn, oracle, N, L, C, G, dtype, silu, affine):
    print("case N=%d L=%d C=%d G=%d %s silu=%d affine=%d" % (N, L, C, G, dtype, silu, affine),
          flush=True)
    from gn_inputs import bf16_bits_to_f32, make_custom
    dev = torch.device("cuda:0")
    x, gamma, beta = make_custom(N, L, C, seed=N * 31 + L + C + G, mean_range=(-2, 2),
                                 std_range=(0.5, 2.0), affine=affine, dtype=dtype)
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    xd = t.to(dev).reshape(N, L, C)
    y = torch.empty_like(xd)
    g = None if gamma is None else torch.from_numpy(gamma).to(dev)
    b = None if beta is None else torch.from_numpy(beta).to(dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    code = gn.gn_silu_rows_dtype(vp(xd), vp(g), vp(b), vp(y), N, L, C, G, 1e-6, silu,
                                 CODE[dtype], stream)
    assert code == gn.GnStatus.OK, gn.status_text(code)
    torch.cuda.synchronize()
    ref = oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, silu,
                         out_dtype=np.float32).reshape(-1)
    if dtype == "bf16":
        got_all = y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    else:
        got_all = y.contiguous().cpu().numpy().reshape(-1)
    atol, rtol = TOL[dtype]
    bad, worst, first = 0, 0.0, None
    step = 1 << 24
    for s in range(0, ref.size, step):
        gpart = got_all[s:s + step]
        got = (bf16_bits_to_f32(gpart) if dtype == "bf16" else gpart).astype(np.float64)
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
    print("max|y-ref|=%.3e violations=%d/%d first=%s" % (worst, bad, ref.size, first), flush=True)
    assert bad == 0, "%d elements outside tolerance, first %s" % (bad, first)

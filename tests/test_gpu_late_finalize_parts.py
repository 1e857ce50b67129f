"""GPU parity of the late finalize's threads that hold no part of the sum.

In the late finalize every step-3 workgroup reduces its sample's chunk
partials itself: thread tid = g + G*j adds chunks j, j + tpg, ... (tpg =
256 // G).  Threads whose part would be empty still load a batch of partials
(part 0's) and add none of them, so that no load of the prologue sits under a
branch on the thread index; that concerns the parts j >= K1 (fewer step-1
chunks than parts) and, when G does not divide 256, the threads past tpg*G.
These cases reach both kinds, in all three element types, with power-of-two
and other channel counts.  Each output element is compared with the fp64
oracle at the parity tolerances, and the output with gamma/beta held in bf16
(read through their aligned 32-bit words) is compared bit for bit with the
output given the same values in fp32, also with one of the two absent.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

TOL = {"bf16": (1e-2, 1.6e-2), "f16": (1e-4, 1e-3), "f32": (2e-4, 2e-4)}
CODE = {"bf16": 0, "f16": 1, "f32": 2}
ESIZE = {"bf16": 2, "f16": 2, "f32": 4}
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
AFFINE_BF16 = 0x20

CASES = [  # N, L, C, G, dtype
    (1, 4096, 128, 4, "bf16"),    # K1 = 32 chunks for 64 parts per group
    (2, 2048, 120, 12, "f16"),    # both: K1 = 16 < 21 parts, 4 threads past 21*12
    (1, 8192, 96, 24, "bf16"),    # 16 threads past 10*24
    (1, 4096, 240, 40, "f32"),    # 16 threads past 6*40
    (1, 4096, 320, 20, "bf16"),   # 16 threads past 12*20, 320 channels
]


def kinds_of(N, L, C, G, dtype, gn):
    p = gn.plan_rows(N, L, C, G, CODE[dtype])
    tpg = 256 // G
    out = set()
    if p["K1"] < tpg:
        out.add("parts past K1")
    if tpg * G < 256:
        out.add("threads past tpg*G")
    return p, out


def test_cases_reach_the_empty_parts():
    """Every case takes the late finalize in three steps (not the single
    launch), and together they reach both kinds of empty part."""
    import groupnorm_silu_normalization_amd as gn
    seen = set()
    for N, L, C, G, dtype in CASES:
        p, k = kinds_of(N, L, C, G, dtype, gn)
        assert p is not None and p["late_finalize"], (N, L, C, G, dtype)
        assert not gn.plan_single_launch(N, L, C, G, CODE[dtype])["single_launch"]
        assert k, (N, L, C, G, dtype)
        seen |= k
    assert seen == {"parts past K1", "threads past tpg*G"}


@pytest.fixture(scope="module")
def gn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import groupnorm_silu_normalization_amd as g
    return g


def vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def to_f32(y, dtype):
    from gn_inputs import bf16_bits_to_f32
    if dtype == "bf16":
        return bf16_bits_to_f32(y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return y.contiguous().cpu().numpy().astype(np.float32)


@pytest.mark.gpu
@pytest.mark.parametrize("N,L,C,G,dtype", CASES)
def test_empty_parts_against_the_oracle(gn, oracle, N, L, C, G, dtype):
    print("case N=%d L=%d C=%d G=%d %s" % (N, L, C, G, dtype), flush=True)
    from gn_inputs import make_custom
    dev = torch.device("cuda:0")
    x, gamma, beta = make_custom(N, L, C, seed=7 * N + L + C + G, mean_range=(-2, 2),
                                 std_range=(0.5, 2.0), affine=True, dtype=dtype)
    # gamma/beta rounded to bf16, so the bf16 copies hold the same values
    gamma = torch.from_numpy(gamma).to(torch.bfloat16).float().numpy()
    beta = torch.from_numpy(beta).to(torch.bfloat16).float().numpy()
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    xd = t.to(dev).reshape(N, L, C)
    g32 = torch.from_numpy(gamma).to(dev)
    b32 = torch.from_numpy(beta).to(dev)
    g16, b16 = g32.to(torch.bfloat16), b32.to(torch.bfloat16)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def run(g, b, flag, silu):
        y = torch.empty_like(xd)
        code = gn.gn_silu_rows_dtype(vp(xd), vp(g), vp(b), vp(y), N, L, C, G, 1e-6, silu,
                                     CODE[dtype] | flag, stream)
        assert code == gn.GnStatus.OK, gn.status_text(code)
        return y

    y = run(g32, b32, 0, 1)
    pairs = [(y, run(g16, b16, AFFINE_BF16, 1)),
             (run(g32, None, 0, 0), run(g16, None, AFFINE_BF16, 0)),
             (run(None, b32, 0, 1), run(None, b16, AFFINE_BF16, 1))]
    torch.cuda.synchronize()
    for a, b in pairs:
        assert torch.equal(a.view(-1).view(torch.uint8), b.view(-1).view(torch.uint8))
    ref = oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, 1,
                         out_dtype=np.float32).reshape(-1).astype(np.float64)
    got = to_f32(y, dtype).reshape(-1).astype(np.float64)
    atol, rtol = TOL[dtype]
    err = np.abs(got - ref)
    ok = err <= atol + rtol * np.abs(ref)
    bad = int(np.count_nonzero(~ok))
    print("max|y-ref|=%.3e violations=%d/%d" % (float(np.nanmax(err)), bad, ref.size),
          flush=True)
    assert bad == 0

"""GPU parity of the fused GroupNorm(+SiLU) -> 3x3 convolution on seeded
random problems.

A fixed seed draws 24 problems: N 1-2, H and W from 1 to 96 (tiles cut
anywhere, images smaller than one 8 x 16 tile included), Ci a multiple of 32
up to 1024 (small ones more often, so that larger images fit the oracle's
budget), Co a multiple of 128 up to 1024 (so 256-channel and 128-channel
workgroups, and every XCD block mapping), G any divisor of Ci, G2 any group
count with Co/G2 dividing 64, and one of four variants: the plain conv, the
GroupNorm+SiLU prologue with output statistics, the GroupNorm prologue
without SiLU with a residual and statistics, and the GroupNorm+SiLU prologue
with a residual.  Each is compared with the fp64 oracle under the tolerance
and the rms bound of tests/test_gpu_conv.py (its module docstring derives
them), and the statistics with the bounds propagated there.
"""
import random

import pytest

torch = pytest.importorskip("torch")

from test_gpu_conv import check_stats, compare, make_problem, run_gpu, tolerance  # noqa: E402

pytestmark = pytest.mark.gpu

VARIANTS = ("plain", "gn_silu_stats", "gn_res_stats", "gn_silu_res")


def draw_problems(seed=1203, count=24):
    rng = random.Random(seed)
    out = []
    while len(out) < count:
        N = rng.choice([1, 1, 2])
        H, W = rng.randrange(1, 97), rng.randrange(1, 97)
        Ci = 32 * rng.choice([1, 1, 2, 2, 3, 4, 6, 8, 13, 16, 32])
        Co = 128 * rng.choice([1, 2, 3, 4, 6, 8])
        if N * H * W * Co * 9 * Ci > 400_000_000:  # keep the fp64 oracle at seconds
            continue
        G = rng.choice([g for g in range(1, Ci + 1) if Ci % g == 0])
        Cg2 = rng.choice([c for c in (1, 2, 4, 8, 16, 32, 64) if Co % c == 0])
        variant = rng.choice(VARIANTS)
        out.append((N, H, W, Ci, Co, G, Co // Cg2, variant))
    return out


PROBLEMS = draw_problems()


@pytest.fixture(scope="module")
def gn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import groupnorm_silu_normalization_amd as g
    return g


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def test_draw_reaches_every_variant_and_both_tiles(gn):
    assert {p[-1] for p in PROBLEMS} == set(VARIANTS)
    grids = [gn.conv_plan(*p[:5], p[6])["grid"] for p in PROBLEMS]
    assert max(grids) >= 48, "some problem spans many workgroups"
    assert min(grids) <= 8
    cos = {p[4] for p in PROBLEMS}
    assert any(c % 256 == 0 for c in cos) and any(c % 256 != 0 for c in cos)
    assert any(p[1] < 8 or p[2] < 16 for p in PROBLEMS), "an image smaller than one tile"


@pytest.mark.parametrize("N,H,W,Ci,Co,G,G2,variant", PROBLEMS)
def test_random_conv_against_the_oracle(gn, dev, oracle, N, H, W, Ci, Co, G, G2, variant):
    print("case %s N=%d H=%d W=%d Ci=%d Co=%d G=%d G2=%d" % (variant, N, H, W, Ci, Co, G, G2),
          flush=True)
    seed = N * 1000003 + H * 1009 + W * 101 + Ci + Co
    res = variant in ("gn_res_stats", "gn_silu_res")
    x, gamma, beta, wb, bias, r = make_problem(N, H, W, Ci, Co, seed=seed, res=res)
    if variant == "plain":
        z, _, _ = run_gpu(gn, dev, N, H, W, Ci, Co, x, None, None, wb, bias, None, G, False,
                          False, None)
        ref, mag = oracle.conv3x3(x, wb, bias, N, H, W, Ci, Co, return_abs=True)
        compare(z, ref, tolerance(ref, mag, Ci, False), variant)
        return
    silu = variant in ("gn_silu_stats", "gn_silu_res")
    stats = variant in ("gn_silu_stats", "gn_res_stats")
    z, m2, r2 = run_gpu(gn, dev, N, H, W, Ci, Co, x, gamma, beta, wb, bias, r, G, silu, True,
                        G2 if stats else None)
    ref, mag, _, _ = oracle.gn_silu_conv3x3(x, gamma, beta, G, 1e-6, silu, wb, bias, N, H, W,
                                            Ci, Co, res=r)
    tol = tolerance(ref, mag, Ci, True)
    compare(z, ref, tol, variant)
    if stats:
        check_stats(m2, r2, ref, tol, N, H * W, Co, G2, 1e-6, variant)

"""Pins for the fp64 oracle, against things other than itself.

The operation is the channels-last GroupNorm with optional SiLU of
"FLUX.2 VAE decoder fast path behind quality=high" (Modifications section 1
"Kernel").  The pages print no element values for it, so the pins are:

  * exact-arithmetic brute force on tiny inputs (Fraction for the statistics,
    60-digit Decimal for sqrt/exp) -- bf16 inputs are dyadic rationals;
  * library routines that compute the same op or a special case of it
    (torch's fp64 CPU group_norm, layer_norm for G=1, instance_norm for G=C);
  * closed forms that separate the plausible readings (biased vs unbiased
    variance, eps inside vs outside the square root, SiLU's definition);
  * invariants (zero mean / known variance after normalisation, constant
    groups, row permutation, scale invariance with eps rescaled).

A dropped term, a wrong sign, a wrong channel->group map, a transposed
operand or a wrong variance estimator fails at least one of these.
"""
import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from gn_inputs import bf16_bits_to_f32, f32_to_bf16_bits, make_custom

pytestmark = pytest.mark.filterwarnings("ignore")


def rand_bits(rng, shape, mean=0.0, std=1.0):
    return f32_to_bf16_bits(rng.normal(mean, std, shape).astype(np.float32))


def dec(fr: Fraction) -> Decimal:
    return Decimal(fr.numerator) / Decimal(fr.denominator)


def exact_reference(x_bits, gamma, beta, N, L, C, G, eps, apply_silu):
    """Brute force in exact rationals (stats) and 60-digit decimals (output)."""
    xs = bf16_bits_to_f32(x_bits).astype(np.float64).reshape(N, L, C)
    Cg = C // G
    means, variances = {}, {}
    out = np.empty((N, L, C), np.float64)
    with localcontext() as ctx:
        ctx.prec = 60
        for n in range(N):
            for g in range(G):
                vals = [Fraction(float(xs[n, l, c]))
                        for l in range(L) for c in range(g * Cg, (g + 1) * Cg)]
                M = len(vals)
                mu = sum(vals, Fraction(0)) / M
                var = sum(((v - mu) ** 2 for v in vals), Fraction(0)) / M
                means[n, g], variances[n, g] = mu, var
                rstd = Decimal(1) / (dec(var) + dec(Fraction(eps))).sqrt()
                for l in range(L):
                    for c in range(g * Cg, (g + 1) * Cg):
                        ga = Decimal(1) if gamma is None else dec(Fraction(float(gamma[c])))
                        be = Decimal(0) if beta is None else dec(Fraction(float(beta[c])))
                        t = ga * ((dec(Fraction(float(xs[n, l, c]))) - dec(mu)) * rstd) + be
                        if apply_silu:
                            t = t / (Decimal(1) + (-t).exp())
                        out[n, l, c] = float(t)
    return out, means, variances


def divisors(c):
    return [g for g in range(1, c + 1) if c % g == 0]


TINY = [(1, 1, 1), (1, 2, 2), (1, 3, 4), (2, 2, 4), (1, 4, 8), (2, 3, 8), (1, 9, 2), (2, 1, 8)]


@pytest.mark.parametrize("N,L,C", TINY)
def test_exact_bruteforce_stats_and_output(oracle, N, L, C):
    rng = np.random.default_rng(100 + 7 * N + 3 * L + C)
    for G in divisors(C):
        for mean, std in ((0.0, 1.0), (3.0, 0.05), (-40.0, 2.0)):
            x = rand_bits(rng, N * L * C, mean, std)
            gamma = rng.normal(1.0, 0.3, C).astype(np.float32)
            beta = rng.normal(0.0, 0.3, C).astype(np.float32)
            eps = 1e-5
            for silu in (False, True):
                y, m, v = oracle.gn_silu(x, gamma, beta, N, L, C, G, eps, silu,
                                         return_stats=True)
                ref, em, ev = exact_reference(x, gamma, beta, N, L, C, G, eps, silu)
                for (n, g), mu in em.items():
                    assert abs(m[n, g] - float(mu)) <= 1e-15 * max(1.0, abs(float(mu)))
                    assert abs(v[n, g] - float(ev[n, g])) <= 1e-13 * max(1e-30, float(ev[n, g])) + 1e-15 * float(mu) ** 2
                np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-10)


def torch_reference(x_bits, gamma, beta, N, L, C, G, eps, apply_silu):
    x = torch.from_numpy(bf16_bits_to_f32(x_bits).astype(np.float64)).reshape(N, L, C)
    xt = x.permute(0, 2, 1).contiguous()  # (N, C, L): the layout torch's GroupNorm expects
    w = None if gamma is None else torch.from_numpy(gamma.astype(np.float64))
    b = None if beta is None else torch.from_numpy(beta.astype(np.float64))
    y = F.group_norm(xt, G, w, b, eps)
    if apply_silu:
        y = F.silu(y)
    return y.permute(0, 2, 1).contiguous().numpy()


@pytest.mark.parametrize("N,L,C,G", [
    (1, 64, 128, 32), (2, 37, 64, 8), (1, 100, 32, 32), (3, 17, 16, 1),
    (1, 5, 2048, 32), (2, 33, 256, 64), (1, 257, 8, 2), (1, 3, 12, 3), (2, 10, 6, 3),
])
@pytest.mark.parametrize("silu", [False, True])
def test_torch_group_norm_fp64(oracle, N, L, C, G, silu):
    x, gamma, beta = make_custom(N, L, C, seed=N * 1000 + L * 10 + C + G,
                                 mean_range=(-4, 4), std_range=(0.2, 3))
    for eps in (1e-6, 0.25):
        y = oracle.gn_silu(x, gamma, beta, N, L, C, G, eps, silu)
        ref = torch_reference(x, gamma, beta, N, L, C, G, eps, silu)
        np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-11)


def test_no_affine_is_identity_affine(oracle):
    N, L, C, G = 2, 19, 32, 4
    x, _, _ = make_custom(N, L, C, seed=5)
    ones = np.ones(C, np.float32)
    zeros = np.zeros(C, np.float32)
    for silu in (False, True):
        a = oracle.gn_silu(x, None, None, N, L, C, G, 1e-6, silu)
        b = oracle.gn_silu(x, ones, zeros, N, L, C, G, 1e-6, silu)
        assert np.array_equal(a, b)
        ref = torch_reference(x, None, None, N, L, C, G, 1e-6, silu)
        np.testing.assert_allclose(a, ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("N,L,C", [(1, 50, 16), (2, 7, 64), (1, 300, 4)])
def test_layer_norm_identity_g1(oracle, N, L, C):
    """G = 1: LayerNorm over each sample's (L, C) block, then a per-channel affine."""
    x, gamma, beta = make_custom(N, L, C, seed=77 + C, mean_range=(-2, 2), std_range=(0.5, 2))
    eps = 1e-5
    xf = torch.from_numpy(bf16_bits_to_f32(x).astype(np.float64)).reshape(N, L, C)
    ln = F.layer_norm(xf, (L, C), None, None, eps)
    ref = ln * torch.from_numpy(gamma.astype(np.float64)) + torch.from_numpy(beta.astype(np.float64))
    y = oracle.gn_silu(x, gamma, beta, N, L, C, 1, eps, False)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("N,L,C", [(1, 50, 16), (2, 7, 64), (3, 129, 8)])
def test_instance_norm_identity_gc(oracle, N, L, C):
    """G = C: InstanceNorm of each (n, c) over L, then the affine."""
    x, gamma, beta = make_custom(N, L, C, seed=91 + C, mean_range=(-2, 2), std_range=(0.5, 2))
    eps = 1e-5
    xf = torch.from_numpy(bf16_bits_to_f32(x).astype(np.float64)).reshape(N, L, C).permute(0, 2, 1)
    inn = F.instance_norm(xf.contiguous(), weight=torch.from_numpy(gamma.astype(np.float64)),
                          bias=torch.from_numpy(beta.astype(np.float64)), eps=eps)
    y = oracle.gn_silu(x, gamma, beta, N, L, C, C, eps, True)
    np.testing.assert_allclose(y, F.silu(inn).permute(0, 2, 1).numpy(), rtol=1e-11, atol=1e-11)


def test_closed_form_biased_variance_and_eps_inside_sqrt(oracle):
    """One group holding {1, 2, 3, 4} (as two rows of two channels, G=1).

    mean = 5/2, biased variance = 5/4 (the unbiased one would be 5/3).
    With eps = 11/4 the denominator is sqrt(5/4 + 11/4) = 2 exactly, so
    z = (x - 5/2) / 2 = {-3/4, -1/4, 1/4, 3/4}; eps outside the root would
    give 1/(sqrt(5/4) + 11/4) instead.
    """
    x = f32_to_bf16_bits(np.array([1, 2, 3, 4], np.float32))
    y, m, v = oracle.gn_silu(x, None, None, 1, 2, 2, 1, 2.75, False, return_stats=True)
    assert m[0, 0] == 2.5 and v[0, 0] == 1.25
    assert y.reshape(-1).tolist() == [-0.75, -0.25, 0.25, 0.75]


def test_closed_form_affine_and_silu(oracle):
    """Group {-1, +1} per channel pair with eps = 0: z = -1, +1 exactly.

    gamma = (2, 0.5), beta = (0.5, -1): t = gamma*z + beta.
    SiLU(t) = t / (1 + e^-t) is checked against math.exp, and
    SiLU(t) - SiLU(-t) = t against the t = +/-1 entries.
    """
    x = f32_to_bf16_bits(np.array([-1, 1, 1, -1], np.float32))  # rows (l) x channels (c)
    gamma = np.array([2.0, 0.5], np.float32)
    beta = np.array([0.5, -1.0], np.float32)
    t_expected = np.array([2 * -1 + 0.5, 0.5 * 1 - 1, 2 * 1 + 0.5, 0.5 * -1 - 1])
    t = oracle.gn_silu(x, gamma, beta, 1, 2, 2, 1, 0.0, False).reshape(-1)
    assert t.tolist() == t_expected.tolist()
    y = oracle.gn_silu(x, gamma, beta, 1, 2, 2, 1, 0.0, True).reshape(-1)
    for got, tv in zip(y, t_expected):
        assert got == pytest.approx(tv / (1.0 + math.exp(-tv)), rel=1e-15, abs=1e-300)
    # the odd part of SiLU is the identity: SiLU(1) - SiLU(-1) = 1
    xs = f32_to_bf16_bits(np.array([-1, 1], np.float32))
    s = oracle.gn_silu(xs, None, None, 1, 2, 1, 1, 0.0, True).reshape(-1)
    assert s[1] - s[0] == pytest.approx(1.0, rel=1e-15)
    assert s[1] == pytest.approx(math.e / (math.e + 1.0), rel=1e-15)


def test_silu_limits(oracle):
    """SiLU(0) = 0; SiLU(t) -> t for large t; -> -0 (not NaN) for t << 0."""
    beta = np.array([0.0, 60.0, -800.0], np.float32)
    x = f32_to_bf16_bits(np.zeros(3, np.float32))  # constant groups: z = 0, t = beta
    y = oracle.gn_silu(x, np.ones(3, np.float32), beta, 1, 1, 3, 3, 1e-6, True).reshape(-1)
    assert y[0] == 0.0
    assert y[1] == pytest.approx(60.0, rel=1e-15)
    assert y[2] == 0.0 and not np.isnan(y[2])


def test_constant_group_gives_beta(oracle):
    """Zero variance: every output of the group equals beta_c (then SiLU of it)."""
    N, L, C, G = 2, 13, 16, 4
    x = f32_to_bf16_bits(np.full(N * L * C, 3.25, np.float32))
    gamma = np.linspace(0.5, 2, C).astype(np.float32)
    beta = np.linspace(-1, 1, C).astype(np.float32)
    y = oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, False)
    assert np.array_equal(y, np.broadcast_to(beta.astype(np.float64), (N, L, C)))
    ys = oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, True)
    b = beta.astype(np.float64)
    np.testing.assert_allclose(ys, np.broadcast_to(b / (1 + np.exp(-b)), (N, L, C)), rtol=1e-15)


@pytest.mark.parametrize("mean", [0.0, 8.0, -100.0])
def test_normalised_moments(oracle, mean):
    """gamma=1, beta=0, no SiLU: each group has mean 0 and variance var/(var+eps)."""
    N, L, C, G = 2, 200, 32, 8
    x, _, _ = make_custom(N, L, C, seed=int(mean) + 500, mean_range=(mean - 1, mean + 1),
                          std_range=(0.25, 1))
    eps = 1e-2
    y, m, v = oracle.gn_silu(x, None, None, N, L, C, G, eps, False, return_stats=True)
    Cg = C // G
    for n in range(N):
        for g in range(G):
            blk = y[n, :, g * Cg:(g + 1) * Cg]
            assert abs(blk.mean()) < 1e-12
            assert blk.var() == pytest.approx(v[n, g] / (v[n, g] + eps), rel=1e-12)


def test_row_permutation_equivariance(oracle):
    N, L, C, G = 1, 64, 32, 8
    x, gamma, beta = make_custom(N, L, C, seed=3, mean_range=(-1, 1))
    perm = np.random.default_rng(4).permutation(L)
    xp = x.reshape(N, L, C)[:, perm, :].reshape(-1).copy()
    y = oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-6, True)
    yp = oracle.gn_silu(xp, gamma, beta, N, L, C, G, 1e-6, True)
    np.testing.assert_allclose(yp, y[:, perm, :], rtol=1e-13, atol=1e-13)


def test_scale_and_shift_invariance(oracle):
    """GN(a*x + b) with eps*a^2 equals GN(x) with eps (a = 4, b = 1, exact in bf16)."""
    N, L, C, G = 1, 40, 16, 4
    rng = np.random.default_rng(9)
    xi = rng.integers(-8, 9, N * L * C).astype(np.float32)
    x = f32_to_bf16_bits(xi)
    x2 = f32_to_bf16_bits(4 * xi + 1)
    assert np.array_equal(bf16_bits_to_f32(x2), 4 * xi + 1)
    gamma = rng.normal(1, 0.2, C).astype(np.float32)
    beta = rng.normal(0, 0.2, C).astype(np.float32)
    a = oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-3, True)
    b = oracle.gn_silu(x2, gamma, beta, N, L, C, G, 16e-3, True)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_empty_inputs(oracle):
    for N, L in ((0, 5), (3, 0), (0, 0)):
        y = oracle.gn_silu(np.zeros(0, np.uint16), None, None, N, L, 8, 2, 1e-6, True)
        assert y.shape == (N, L, 8)


def test_rejects_bad_shapes(oracle):
    x = np.zeros(12, np.uint16)
    with pytest.raises(ValueError):
        oracle.gn_silu(x, None, None, 1, 2, 6, 4, 1e-6, True)  # C % G != 0
    with pytest.raises(ValueError):
        oracle.gn_silu(x, None, None, 1, 2, 6, 0, 1e-6, True)  # G = 0
    with pytest.raises(ValueError):
        oracle.gn_silu(x, None, None, 1, 2, 6, 3, -1.0, True)  # eps < 0


def test_input_generator_recipe():
    """The shared generator's bf16 rounding is round-to-nearest-even."""
    v = np.array([1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -9, -3.0e-3], np.float32)
    bits = f32_to_bf16_bits(v)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties to even gives 1.0
    assert bf16_bits_to_f32(bits).tolist()[:2] == [1.0, 1.0]
    # 1 + 3*2^-9 lies above the midpoint 1 + 2^-8: rounds up to 1 + 2^-7
    assert bf16_bits_to_f32(bits)[2] == np.float32(1.0078125)
    # exactly torch's bf16 rounding
    t = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, t)


def test_widen_bf16_exhaustive(oracle):
    """All 65536 bf16 patterns widen exactly as torch's bf16 -> float64."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen(bits)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    assert (np.signbit(got) == np.signbit(want))[~np.isnan(want)].all()


def test_widen_f16_exhaustive(oracle):
    """All 65536 binary16 patterns (subnormals, infinities, NaNs included)
    widen exactly as numpy's float16 -> float64."""
    vals = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    got = oracle.widen(vals)
    want = vals.astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    assert (np.signbit(got) == np.signbit(want))[~np.isnan(want)].all()


def test_widen_f32_is_identity(oracle):
    v = np.random.default_rng(1).normal(0, 1e3, 4096).astype(np.float32)
    v[:4] = [np.inf, -np.inf, 1e-45, -0.0]
    assert np.array_equal(oracle.widen(v), v.astype(np.float64))


@pytest.mark.parametrize("dtype", ["float16", "float32"])
def test_torch_group_norm_other_dtypes(oracle, dtype):
    """fp16 and fp32 inputs: the same fp64 GroupNorm(+SiLU) as torch's."""
    rng = np.random.default_rng(123)
    for (N, L, C, G) in ((2, 37, 64, 8), (1, 100, 128, 32), (3, 9, 6, 3)):
        x = (rng.normal(0, 2, (N, L, C)) + rng.uniform(-5, 5, C)).astype(dtype)
        gamma = rng.normal(1, 0.2, C).astype(np.float32)
        beta = rng.normal(0, 0.2, C).astype(np.float32)
        for silu in (False, True):
            y = oracle.gn_silu(x, gamma, beta, N, L, C, G, 1e-5, silu)
            xt = torch.from_numpy(x.astype(np.float64)).permute(0, 2, 1).contiguous()
            ref = F.group_norm(xt, G, torch.from_numpy(gamma.astype(np.float64)),
                               torch.from_numpy(beta.astype(np.float64)), 1e-5)
            if silu:
                ref = F.silu(ref)
            np.testing.assert_allclose(y, ref.permute(0, 2, 1).numpy(), rtol=1e-11, atol=1e-11)

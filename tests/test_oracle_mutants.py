"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), compiles it with the same flags, and runs a
battery of the pins from ``test_oracle_pins`` against it.  At least one pin
must fail for every mutant, and none may fail for the unmodified source.
"""
import os
import subprocess

import pytest

import oracle as oracle_pkg
import test_oracle_conv_pins as cpins
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle_pkg.__file__), "gn_oracle.c")

MUTANTS = {
    "unbiased variance": ("var_out[ng] = (M > 0) ? ss / (double)M : 0.0;",
                          "var_out[ng] = (M > 1) ? ss / (double)(M - 1) : 0.0;"),
    "eps outside the square root": ("1.0 / sqrt(var[n * G + g] + eps)",
                                    "1.0 / (sqrt(var[n * G + g]) + eps)"),
    "beta dropped": ("((xv - mu) * rstd) + be;", "((xv - mu) * rstd);"),
    "gamma dropped": ("const double t = ga * ((xv - mu) * rstd) + be;",
                      "const double t = ((xv - mu) * rstd) + be;"),
    "mean added instead of subtracted": ("(xv - mu)", "(xv + mu)"),
    "channel->group map by modulo": ("const int64_t g = c / Cg;", "const int64_t g = c % G;"),
    "SiLU with the wrong sign": ("t / (1.0 + exp(-t))", "t / (1.0 + exp(t))"),
    "group offset dropped in stats": ("const int64_t base = n * L * C + g * Cg;",
                                      "const int64_t base = n * L * C + g;"),
    "row stride Cg instead of C in the mean": (
        "sum += load(x, dtype, base + l * C + j);",
        "sum += load(x, dtype, base + l * Cg + j);"),
    "second moment not centred": (
        "const double d = load(x, dtype, base + l * C + j) - mu;",
        "const double d = load(x, dtype, base + l * C + j);"),
    "fp16 exponent bias off by one": ("ldexp((double)(f + 1024), e - 25)",
                                      "ldexp((double)(f + 1024), e - 24)"),
    "fp16 subnormal scale wrong": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "fp16 implicit bit dropped": ("ldexp((double)(f + 1024), e - 25)",
                                  "ldexp((double)f, e - 25)"),
    "sample index ignored": ("const int64_t n = row / L;", "const int64_t n = 0;"),
    "conv: true convolution (taps flipped)": ("const int64_t ih = h + kh - 1;",
                                              "const int64_t ih = h - kh + 1;"),
    "conv: column offset off by one": ("const int64_t iw = w + kw - 1;",
                                       "const int64_t iw = w + kw - 2;"),
    "conv: weight taps transposed": ("wt + ((co * 3 + kh) * 3 + kw) * Ci",
                                     "wt + ((co * 3 + kw) * 3 + kh) * Ci"),
    "conv: bias dropped": ("double acc = bias ? bias[co] : 0.0;", "double acc = 0.0;"),
    "conv: residual dropped": ("acc += res[pix * Co + co];", "acc += 0.0;"),
    "conv: magnitude of negative terms lost": ("mag += fabs(term);", "mag += term;"),
    "fp64 statistics read as fp32": ("if (dtype == GNO_F64) return ((const double *)x)[i];",
                                     "if (dtype == GNO_F64) return ((const float *)x)[i];"),
}


def battery():
    return [
        ("bruteforce", lambda o: pins.test_exact_bruteforce_stats_and_output(o, 2, 2, 4)),
        ("torch_gn", lambda o: pins.test_torch_group_norm_fp64(o, 2, 37, 64, 8, True)),
        ("torch_gn_nosilu", lambda o: pins.test_torch_group_norm_fp64(o, 1, 64, 128, 32, False)),
        ("closed_var_eps", pins.test_closed_form_biased_variance_and_eps_inside_sqrt),
        ("closed_affine_silu", pins.test_closed_form_affine_and_silu),
        ("moments", lambda o: pins.test_normalised_moments(o, 8.0)),
        ("constant_group", pins.test_constant_group_gives_beta),
        ("widen_f16", pins.test_widen_f16_exhaustive),
        ("torch_gn_f16", lambda o: pins.test_torch_group_norm_other_dtypes(o, "float16")),
        ("conv_torch", lambda o: cpins.test_conv_against_torch_fp64(o, 1, 9, 4, 8, 16, True,
                                                                    True)),
        ("conv_exact", cpins.test_conv_exact_integer_bruteforce),
        ("conv_shift", lambda o: cpins.test_conv_off_centre_tap_is_a_shift_with_zero_fill(
            o, 0, 2)),
        ("conv_layout", cpins.test_conv_weight_layout_maps_input_to_output_channels),
        ("conv_abs", cpins.test_conv_magnitude_sum_is_conv_of_absolute_values),
        ("stats_f64", cpins.test_group_stats_of_fp64_input),
    ]


def build_variant(tmp_path, name, source):
    c = tmp_path / (name + ".c")
    so = tmp_path / (name + ".so")
    c.write_text(source)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", "-o", str(so), str(c), "-lm"], check=True)
    return oracle_pkg.Oracle(str(so))


def failing_pins(o):
    failed = []
    for name, fn in battery():
        try:
            fn(o)
        except Exception:  # an assertion, or a shape the mutant gets wrong
            failed.append(name)
    return failed


def test_unmodified_source_passes_battery(tmp_path):
    o = build_variant(tmp_path, "original", open(SRC).read())
    assert failing_pins(o) == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, mutant):
    old, new = MUTANTS[mutant]
    src = open(SRC).read()
    assert old in src, "mutation target no longer in the oracle source: %r" % old
    o = build_variant(tmp_path, "mutant", src.replace(old, new))
    assert failing_pins(o), "no pin caught the planted mistake: " + mutant

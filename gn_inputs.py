"""Seeded synthetic inputs for channels-last GroupNorm(+SiLU).

This module is the only thing the GPU path's tests and the fp64 oracle share.
It draws random numbers and rounds them to bf16 (or fp16); it holds none of the
normalisation arithmetic.

The five workload shapes are the FLUX.2 VAE decoder norm shapes of the kernel
microbenchmark table in "FLUX.2 VAE decoder fast path behind quality=high"
(Speedup section), with G=32.  The pages measure on decoder activations of
frozen latents, which need trained weights; these seeded tensors of the same
shapes stand in for them.  Recipe (fixed draw order, one generator per case):

    rng = numpy.random.default_rng(seed)
    m[C]  per-channel mean   (distribution per case; "zero" draws nothing)
    s[C]  per-channel std    (distribution per case; "one" draws nothing)
    gamma[C] ~ N(1, 0.1), beta[C] ~ N(0, 0.1)          (float32)
    z[N*H*W*C] standard normal float32, NHWC order
    x = bf16_rne(m[c] + s[c] * z)                        (computed in float32)

WIDE_WORKLOADS are shapes outside the pages' kernel's support set (channel
counts that are not powers of two or exceed 2048, and a 5-D NDHWC video-VAE
activation), at sizes of the same order as the decoder shapes.  The pages
give no workload for them: the channel counts are the widths of common
diffusion UNets and their skip concatenations (320, 960, 1280, 2560), and
the 5-D shape is a channels_last_3d activation of D = 9 frames, the kind of
HunyuanVAE-style call site the pages leave on the older kernel.  Same recipe.
"""
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    C: int
    H: int
    W: int
    G: int = 32
    eps: float = 1e-6
    apply_silu: bool = True
    mean_dist: tuple = ("zero",)
    std_dist: tuple = ("one",)
    seed: int = 0
    note: str = field(default="", compare=False)
    D: int = 1          # depth (frames) of a 5-D NDHWC activation; 1 for 4-D

    @property
    def L(self) -> int:
        return self.D * self.H * self.W

    @property
    def numel(self) -> int:
        return self.N * self.C * self.L

    @property
    def algorithmic_bytes(self) -> int:
        # two reads and one write of the bf16 tensor
        return 3 * 2 * self.numel

    def label(self) -> str:
        if self.D != 1:
            return "(%d,%d,%d,%d,%d) G=%d" % (self.N, self.C, self.D, self.H, self.W, self.G)
        return "(%d,%d,%d,%d) G=%d" % (self.N, self.C, self.H, self.W, self.G)


# The five decoder shapes.  Index 0 is the small case the oracle finishes in
# well under a second; indices 2-4 are the >= (1,512,512,512) shapes.
WORKLOADS = (
    Workload("gn_silu_1x128x64x64", 1, 128, 64, 64, seed=1001,
             mean_dist=("zero",), std_dist=("one",),
             note="x ~ N(0,1)"),
    Workload("gn_silu_1x512x128x128", 1, 512, 128, 128, seed=1002,
             mean_dist=("normal", 0.0, 1.0), std_dist=("uniform", 0.5, 2.0),
             note="per-channel mean ~ N(0,1), std ~ U(0.5,2)"),
    Workload("gn_silu_1x512x512x512", 1, 512, 512, 512, seed=1003,
             mean_dist=("zero",), std_dist=("uniform", 0.5, 2.0),
             note="per-channel std ~ U(0.5,2)"),
    Workload("gn_silu_1x256x1024x1024", 1, 256, 1024, 1024, seed=1004,
             mean_dist=("zero",), std_dist=("uniform", 0.5, 2.0),
             note="per-channel std ~ U(0.5,2)"),
    Workload("gn_silu_1x128x1024x1024", 1, 128, 1024, 1024, seed=1005,
             mean_dist=("uniform", -8.0, 8.0), std_dist=("uniform", 0.25, 1.0),
             note="per-channel mean ~ U(-8,8), std ~ U(0.25,1): fp32 cancellation stress"),
)


# Shapes beyond the pages' support set (see the module docstring).
WIDE_WORKLOADS = (
    Workload("gn_silu_1x320x512x512", 1, 320, 512, 512, seed=2001,
             mean_dist=("normal", 0.0, 1.0), std_dist=("uniform", 0.5, 2.0),
             note="UNet width 320; per-channel mean ~ N(0,1), std ~ U(0.5,2)"),
    Workload("gn_silu_1x960x256x256", 1, 960, 256, 256, seed=2002,
             mean_dist=("zero",), std_dist=("uniform", 0.5, 2.0),
             note="skip concatenation 640+320"),
    Workload("gn_silu_1x1280x256x256", 1, 1280, 256, 256, seed=2003,
             mean_dist=("uniform", -8.0, 8.0), std_dist=("uniform", 0.25, 1.0),
             note="UNet width 1280; mean ~ U(-8,8), std ~ U(0.25,1): cancellation stress"),
    Workload("gn_silu_1x2560x128x128", 1, 2560, 128, 128, seed=2004,
             mean_dist=("zero",), std_dist=("uniform", 0.5, 2.0),
             note="skip concatenation 1280+1280, C > 2048"),
    Workload("gn_silu_1x128x9x256x256", 1, 128, 256, 256, D=9, seed=2005,
             mean_dist=("normal", 0.0, 1.0), std_dist=("uniform", 0.5, 2.0),
             note="5-D NDHWC, 9 frames"),
)

# Shapes measured beside the decoder shapes, not part of the metric: the
# pages' (1,512,256,256) decoder norm shape, the attention-style rows call
# (N, L, C) = (1, 16384, 512) with SiLU off (H = L, W = 1), and one GPU's share
# of the (1,256,1024,1024) activation split eight ways along its rows.
EXTRA_WORKLOADS = (
    Workload("gn_silu_1x512x256x256", 1, 512, 256, 256, seed=1006,
             mean_dist=("zero",), std_dist=("uniform", 0.5, 2.0),
             note="per-channel std ~ U(0.5,2)"),
    Workload("gn_rows_1x16384x512_nosilu", 1, 512, 16384, 1, apply_silu=False, seed=1007,
             mean_dist=("normal", 0.0, 1.0), std_dist=("uniform", 0.5, 2.0),
             note="rows (N, L, C) = (1, 16384, 512), SiLU off"),
    Workload("gn_silu_1x256x128x1024_shard", 1, 256, 128, 1024, seed=1008,
             mean_dist=("zero",), std_dist=("uniform", 0.5, 2.0),
             note="1/8 of the rows of (1,256,1024,1024): one GPU's share"),
)


def _draw(rng, dist, C, default):
    kind = dist[0]
    if kind in ("zero", "one"):
        return np.full(C, default, np.float32)
    if kind == "normal":
        return rng.normal(dist[1], dist[2], C).astype(np.float32)
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], C).astype(np.float32)
    raise ValueError("unknown distribution %r" % (dist,))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  Inputs here are finite.
    """
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    step = 1 << 24
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    for s in range(0, flat_u.size, step):
        b = flat_u[s:s + step]
        r = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        flat_o[s:s + step] = ((b + r) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _finish(z, dtype):
    """The float32 draws rounded to the requested element type: bf16 bit
    patterns (uint16), IEEE float16 (round to nearest even) or float32."""
    if dtype == "bf16":
        return f32_to_bf16_bits(z)
    if dtype == "f16":
        return z.astype(np.float16)
    if dtype == "f32":
        return z
    raise ValueError("dtype must be bf16, f16 or f32")


def make_inputs(w: Workload, seed=None, dtype="bf16"):
    """Returns (x [N*H*W*C] in NHWC order, gamma f32[C], beta f32[C]).

    x holds bf16 bit patterns (uint16) by default, or float16 / float32
    values for dtype "f16" / "f32" (the same float32 draws, rounded once).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    C = w.C
    m = _draw(rng, w.mean_dist, C, 0.0)
    s = _draw(rng, w.std_dist, C, 1.0)
    gamma = rng.normal(1.0, 0.1, C).astype(np.float32)
    beta = rng.normal(0.0, 0.1, C).astype(np.float32)
    z = rng.standard_normal(w.numel, dtype=np.float32)
    z2 = z.reshape(-1, C)
    z2 *= s
    z2 += m
    x = _finish(z, dtype)
    del z2
    return x, gamma, beta


def make_custom(N, L, C, seed, mean_range=(0.0, 0.0), std_range=(1.0, 1.0),
                affine=True, dtype="bf16"):
    """Seeded [N, L, C] input of any shape for parity sweeps.

    Per-channel mean ~ U(mean_range), std ~ U(std_range), then the same
    gamma/beta/z draws as ``make_inputs``; x in the element type `dtype`.
    """
    rng = np.random.default_rng(seed)
    m = rng.uniform(mean_range[0], mean_range[1], C).astype(np.float32)
    s = rng.uniform(std_range[0], std_range[1], C).astype(np.float32)
    gamma = rng.normal(1.0, 0.1, C).astype(np.float32)
    beta = rng.normal(0.0, 0.1, C).astype(np.float32)
    z = rng.standard_normal(N * L * C, dtype=np.float32)
    if z.size:
        z2 = z.reshape(-1, C)
        z2 *= s
        z2 += m
    x = _finish(z, dtype)
    if not affine:
        gamma = beta = None
    return x, gamma, beta

"""GroupNorm weight and bias held in bf16 or fp16 (GN_AFFINE_BF16 / GN_AFFINE_F16).

A decoder cast to bf16 or fp16 holds its GroupNorm weight and bias in that
type.  The library widens each value exactly to fp32 before folding it into
scale/shift, so the output with 16-bit gamma/beta must equal, bit for bit,
the output with fp32 gamma/beta holding the same values (every 16-bit value
is exactly representable in fp32), and must lie within the parity tolerance
of the oracle's fp64 GroupNorm of those values.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-2, 1.6e-2


@pytest.fixture(scope="module")
def gn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import groupnorm_silu_normalization_amd as gn
    return gn


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def bits(t):
    """The raw bits of a tensor, for bitwise comparison."""
    return t.contiguous().view({2: torch.int16, 4: torch.int32}[t.element_size()])


def make(dev, N, C, H, W, G, xdt, adt, seed):
    gen = torch.Generator().manual_seed(seed)
    x = (torch.randn(N, C, H, W, generator=gen) * 1.5 + 0.25).to(xdt)
    x = x.to(dev).contiguous(memory_format=torch.channels_last)
    g = (1.0 + 0.3 * torch.randn(C, generator=gen)).to(adt).to(dev)
    b = (0.2 * torch.randn(C, generator=gen)).to(adt).to(dev)
    return x, g, b


SHAPES = [  # N, C, H, W, G; the last three take the single launch (gn_strip)
    (1, 128, 64, 64, 32), (2, 320, 24, 40, 32), (1, 2560, 16, 16, 32), (1, 512, 128, 128, 32),
    (3, 96, 7, 9, 24), (2, 256, 32, 32, 32), (4, 128, 32, 32, 32),
]


@pytest.mark.parametrize("adt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("shape", SHAPES)
def test_16bit_affine_equals_fp32_affine(gn, dev, shape, xdt, adt):
    N, C, H, W, G = shape
    print("case 4d N=%d C=%d H=%d W=%d G=%d x=%s affine=%s" % (N, C, H, W, G, xdt, adt),
          flush=True)
    x, g, b = make(dev, N, C, H, W, G, xdt, adt, seed=C + H)
    with torch.no_grad():
        y16 = gn.group_norm_silu_4d(x, G, g, b, 1e-6)
        y32 = gn.group_norm_silu_4d(x, G, g.float(), b.float(), 1e-6)
        # one of the two absent: 1 / 0 in its place
        yg16 = gn.group_norm_silu_4d(x, G, g, None, 1e-6, apply_silu=False)
        yg32 = gn.group_norm_silu_4d(x, G, g.float(), None, 1e-6, apply_silu=False)
        yb16 = gn.group_norm_silu_4d(x, G, None, b, 1e-6)
        yb32 = gn.group_norm_silu_4d(x, G, None, b.float(), 1e-6)
    for a in (y16, y32, yg16, yg32, yb16, yb32):
        assert a is not None
    assert torch.equal(bits(y16), bits(y32))
    assert torch.equal(bits(yg16), bits(yg32))
    assert torch.equal(bits(yb16), bits(yb32))


def test_single_launch_shapes_listed(gn):
    """The shapes above reach both the single launch and the three steps."""
    single = [gn.plan_single_launch(N, H * W, C, G, 0)["single_launch"]
              for N, C, H, W, G in SHAPES]
    assert any(single) and not all(single)


@pytest.mark.parametrize("adt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("shape", [(3, 96, 7, 9, 24), (2, 256, 32, 32, 32),
                                   (1, 512, 128, 128, 32), (2, 320, 24, 40, 32)])
def test_16bit_affine_at_an_odd_element_offset(gn, dev, shape, adt):
    """16-bit gamma/beta need only 2-byte alignment: views one element into
    a buffer (addresses 2 mod 4) give, bit for bit, the output of fp32 copies
    of the same values, in the single launch and in the three steps."""
    N, C, H, W, G = shape
    print("case odd offset N=%d C=%d H=%d W=%d G=%d affine=%s" % (N, C, H, W, G, adt),
          flush=True)
    x, g, b = make(dev, N, C, H, W, G, torch.bfloat16, adt, seed=C + W)
    gbuf = torch.empty(C + 1, dtype=adt, device=dev)
    bbuf = torch.empty(C + 1, dtype=adt, device=dev)
    gbuf[1:] = g
    bbuf[1:] = b
    go, bo = gbuf[1:], bbuf[1:]
    assert go.data_ptr() % 4 == 2 and bo.data_ptr() % 4 == 2
    with torch.no_grad():
        y16 = gn.group_norm_silu_4d(x, G, go, bo, 1e-6)
        y32 = gn.group_norm_silu_4d(x, G, g.float(), b.float(), 1e-6)
    assert y16 is not None and y32 is not None
    assert torch.equal(bits(y16), bits(y32))


@pytest.mark.parametrize("adt", [torch.bfloat16, torch.float16])
def test_16bit_affine_rows_5d_and_apply(gn, dev, adt):
    """The rows and 5-D entries and step three alone take the same flag."""
    N, L, C, G = 2, 3000, 256, 32
    gen = torch.Generator().manual_seed(7)
    x = torch.randn(N, L, C, generator=gen).bfloat16().to(dev)
    g = (1.0 + 0.3 * torch.randn(C, generator=gen)).to(adt).to(dev)
    b = (0.2 * torch.randn(C, generator=gen)).to(adt).to(dev)
    with torch.no_grad():
        r16 = gn.group_norm_silu_rows(x, G, g, b, 1e-6)
        r32 = gn.group_norm_silu_rows(x, G, g.float(), b.float(), 1e-6)
        mean, rstd = gn.group_stats_rows(x, G, 1e-6)
        a16 = gn.apply_rows(x, mean, rstd, g, b)
        a32 = gn.apply_rows(x, mean, rstd, g.float(), b.float())
        x5 = torch.randn(1, C, 3, 20, 50, generator=gen).bfloat16().to(dev)
        x5 = x5.contiguous(memory_format=torch.channels_last_3d)
        v16 = gn.group_norm_silu_5d(x5, G, g, b, 1e-6)
        v32 = gn.group_norm_silu_5d(x5, G, g.float(), b.float(), 1e-6)
    for a in (r16, r32, a16, a32, v16, v32):
        assert a is not None
    assert torch.equal(bits(r16), bits(r32))
    assert torch.equal(bits(a16), bits(a32))
    assert torch.equal(bits(r16), bits(a16))  # the same steps either way
    assert torch.equal(bits(v16), bits(v32))


@pytest.mark.parametrize("adt", [torch.bfloat16, torch.float16])
def test_16bit_affine_against_oracle(gn, dev, oracle, adt):
    """bf16 x and 16-bit gamma/beta against the fp64 GroupNorm+SiLU of the
    same (widened) values."""
    from gn_inputs import bf16_bits_to_f32
    N, C, H, W, G = 1, 512, 96, 80, 32
    x, g, b = make(dev, N, C, H, W, G, torch.bfloat16, adt, seed=11)
    with torch.no_grad():
        y = gn.group_norm_silu_4d(x, G, g, b, 1e-6)
    assert y is not None
    torch.cuda.synchronize()
    x_bits = x.permute(0, 2, 3, 1).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    y_bits = y.permute(0, 2, 3, 1).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.gn_silu(x_bits.reshape(-1), g.float().cpu().numpy(), b.float().cpu().numpy(),
                         N, H * W, C, G, 1e-6, True)
    got = bf16_bits_to_f32(y_bits.reshape(-1)).astype(np.float64)
    err = np.abs(got - ref.reshape(-1))
    print("affine %s: max|y-ref|=%.3e" % (adt, float(err.max())), flush=True)
    assert np.all(err <= ATOL + RTOL * np.abs(ref.reshape(-1)))


def test_mixed_affine_types_fall_back(gn, dev):
    """Weight and bias of different types: the binding declines (None)."""
    x, g, b = make(dev, 1, 64, 8, 8, 32, torch.bfloat16, torch.bfloat16, seed=3)
    with torch.no_grad():
        assert gn.group_norm_silu_4d(x, 32, g, b.float(), 1e-6) is None
        assert gn.group_norm_silu_4d(x, 32, g.half(), b, 1e-6) is None
        assert gn.group_norm_silu_4d(x, 32, g.double(), b.double(), 1e-6) is None


def test_affine_flags_through_the_c_abi(gn, dev):
    """The flag on the C entry point: misaligned 16-bit gamma is declined, a
    flag with other bits set is invalid, and a valid call matches fp32."""
    N, L, C, G = 1, 512, 128, 32
    x = torch.randn(N, L, C, device=dev).bfloat16()
    y16, y32 = torch.empty_like(x), torch.empty_like(x)
    g = (1.0 + 0.3 * torch.randn(C + 1, device=dev)).bfloat16()
    b = (0.2 * torch.randn(C, device=dev)).bfloat16()
    s = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    odd = ctypes.c_void_p(g.data_ptr() + 1)
    call = gn.gn_silu_rows_dtype
    assert call(vp(x), odd, vp(b), vp(y16), N, L, C, G, 1e-6, 1, 0x20, s) == gn.GnStatus.UNSUPPORTED
    assert call(vp(x), vp(g), vp(b), vp(y16), N, L, C, G, 1e-6, 1, 0x40, s) == \
        gn.GnStatus.INVALID_ARGUMENT
    assert call(vp(x), vp(g), vp(b), vp(y16), N, L, C, G, 1e-6, 1, 0x20, s) == gn.GnStatus.OK
    gf, bf = g[:C].float(), b.float()
    assert call(vp(x), vp(gf), vp(bf), vp(y32), N, L, C, G, 1e-6, 1, 0x10, s) == gn.GnStatus.OK
    torch.cuda.synchronize()
    assert torch.equal(bits(y16), bits(y32))

"""GPU parity of the fused GroupNorm(+SiLU) -> 3x3 convolution (-> statistics).

The fused operation is the decoder ResnetBlock2D's GroupNorm -> SiLU ->
Conv2d(3x3, p1) chain ("FLUX.2 VAE decoder fast path behind quality=high",
Modifications section 2), with the next GroupNorm's statistics of the conv
output.  Reference: the fp64 oracle (``oracle.gn_silu`` then
``oracle.conv3x3``, or ``oracle.gn_silu_conv3x3``, also at the decoder's full
sizes), which also returns, per output, the sum of the absolute values of
its terms, mag = |bias| + |res| + sum |w * y|.

Tolerance per output element, from the arithmetic (NaN never passes):
  * z is rounded once to bf16:                      2^-9 |z|   (taken as 2^-8 |ref|)
  * products of bf16 operands are exact in fp32; the K + 2 terms
    (K = 9 * Ci) are summed in fp32:                (K + 2) * 2^-24 * mag
  * with the prologue, y is rounded to bf16 before the matrix cores
    (2^-9 relative per term) and is computed from fp32 statistics and an fp32
    transform (< 2^-16 relative):                   (2^-9 + 2^-16) * mag
  * plus 1e-6 absolute.
The output statistics (fp32 mean and rstd per (n, group) of the stored bf16
z) are compared with the oracle's fp64 statistics of its own z, with bounds
propagated from the per-element bound e: |d mean| <= avg(e);
|d var| <= 2 avg(|z - mean| e) + avg(e^2); |d rstd| <= rstd^3 / 2 * |d var|;
each with a relative margin of 1e-5 for the fp32 tile sums and the fp64 merge.

The worst-case bound grows with mag, which exceeds |z| by about sqrt(K), so it
alone would let a small structural mistake through (a dropped tap moves z by
about a third of its size, inside 2^-9 * mag for large Ci).  Every comparison
therefore also bounds the root-mean-square error: the roundings above are
unbiased and independent, about 2^-9 / sqrt(3) = 1.1e-3 of rms(z) each for z
and (with the prologue) y, so rms(err) <= 4e-3 * rms(ref) holds with room,
and a dropped tap or channel fails it by two orders of magnitude.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

U24 = 2.0 ** -24


@pytest.fixture(scope="module")
def gn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import groupnorm_silu_normalization_amd as g
    return g


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def bits_dev(bits, shape, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev) \
        .view(torch.bfloat16).reshape(shape)


def host_f64(t):
    from gn_inputs import bf16_bits_to_f32
    b = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    return bf16_bits_to_f32(b).astype(np.float64)


def make_problem(N, H, W, Ci, Co, seed, res=False, x_mean=(-1.0, 1.0)):
    """x bf16 [N*H*W*Ci] (NHWC), gamma/beta fp32 [Ci], weight bf16 [Co,3,3,Ci],
    bias fp32 [Co], residual bf16 [N*H*W*Co] or None (seeded)."""
    from gn_inputs import f32_to_bf16_bits, make_custom
    x, gamma, beta = make_custom(N, H * W, Ci, seed=seed, mean_range=x_mean,
                                 std_range=(0.5, 2.0))
    rng = np.random.default_rng(seed + 1)
    w = (rng.standard_normal((Co, 3, 3, Ci)) / np.sqrt(9.0 * Ci)).astype(np.float32)
    wb = f32_to_bf16_bits(w)
    bias = rng.normal(0.0, 0.5, Co).astype(np.float32)
    r = None
    if res:
        r, _, _ = make_custom(N, H * W, Co, seed=seed + 2)
    return x, gamma, beta, wb, bias, r


def run_gpu(gn, dev, N, H, W, Ci, Co, x, gamma, beta, wb, bias, r, G, silu, norm, G2, eps2=1e-6):
    xd = bits_dev(x, (N, H, W, Ci), dev).permute(0, 3, 1, 2)
    wd = bits_dev(wb, (Co, 3, 3, Ci), dev).permute(0, 3, 1, 2)
    bd = torch.from_numpy(bias).to(dev)
    rd = None if r is None else bits_dev(r, (N, H, W, Co), dev).permute(0, 3, 1, 2)
    nrm = None
    if norm:
        rows = xd.permute(0, 2, 3, 1).reshape(N, H * W, Ci)
        with torch.no_grad():
            mean, rstd = gn.group_stats_rows(rows, G, 1e-6)
        nrm = (mean, rstd, torch.from_numpy(gamma).to(dev), torch.from_numpy(beta).to(dev))
    with torch.no_grad():
        out = gn.conv3x3(xd, wd, bd, norm=nrm, apply_silu=silu, residual=rd,
                         next_groups=G2, next_eps=eps2)
    assert out is not None, "conv3x3 declined a supported input"
    torch.cuda.synchronize()
    if G2 is None:
        return host_f64(out.permute(0, 2, 3, 1)), None, None
    z, m2, r2 = out
    return host_f64(z.permute(0, 2, 3, 1)), m2.cpu().numpy(), r2.cpu().numpy()


def tolerance(ref, mag, Ci, prologue):
    K = 9 * Ci
    t = 2.0 ** -8 * np.abs(ref) + (K + 2) * U24 * mag + 1e-6
    if prologue:
        t += (2.0 ** -9 + 2.0 ** -16) * mag
    return t


def compare(got, ref, tol, what, rms_frac=4e-3):
    ref = ref.reshape(-1)
    tol = tol.reshape(-1)
    err = np.abs(got - ref)
    rms_e = float(np.sqrt(np.mean(err ** 2))) if err.size else 0.0
    rms_r = float(np.sqrt(np.mean(ref ** 2))) if err.size else 0.0
    print("%s: rms err / rms ref = %.3e" % (what, rms_e / max(rms_r, 1e-30)), flush=True)
    assert rms_e <= rms_frac * rms_r + 1e-6, "%s: rms error %.3e vs rms %.3e" % (what, rms_e, rms_r)
    ok = err <= tol
    bad = int(np.count_nonzero(~ok))
    first = None
    if bad:
        i = int(np.flatnonzero(~ok)[0])
        first = (i, float(got[i]), float(ref[i]), float(tol[i]))
    print("%s: max err/tol=%.3f max|err|=%.3e violations=%d/%d first=%s" % (
        what, float(np.max(err / tol)) if err.size else 0.0, float(err.max()) if err.size else 0,
        bad, ref.size, first), flush=True)
    assert bad == 0, "%s: %d outputs outside tolerance, first %s" % (what, bad, first)


def check_stats(m2, r2, zref, tol, N, L, Co, G2, eps2, what):
    import oracle
    mref, vref = oracle.group_stats(zref.reshape(-1).copy(), N, L, Co, G2)
    zr = zref.reshape(N, L, G2, Co // G2).transpose(0, 2, 1, 3).reshape(N, G2, -1)
    e = tol.reshape(N, L, G2, Co // G2).transpose(0, 2, 1, 3).reshape(N, G2, -1)
    dmean = e.mean(axis=2) + 1e-5 * (np.abs(mref) + np.sqrt(vref)) + 1e-7
    dvar = (2.0 * (np.abs(zr - mref[..., None]) * e).mean(axis=2) + (e * e).mean(axis=2)
            + 1e-5 * vref + 1e-9)
    rref = 1.0 / np.sqrt(vref + eps2)
    drstd = 0.5 * rref ** 3 * dvar * 1.01 + 1e-5 * rref
    em, er = np.abs(m2 - mref), np.abs(r2 - rref)
    print("%s stats: mean err/bound %.3f, rstd err/bound %.3f" % (
        what, float((em / dmean).max()), float((er / drstd).max())), flush=True)
    assert np.all(em <= dmean), "mean out of bound: %s" % what
    assert np.all(er <= drstd), "rstd out of bound: %s" % what


SHAPES = [  # N, H, W, Ci, Co, G, G2
    (1, 8, 16, 32, 128, 8, 32), (2, 13, 21, 64, 128, 32, 32), (1, 32, 48, 128, 256, 32, 32),
    (1, 5, 7, 32, 128, 4, 8), (3, 9, 17, 96, 384, 24, 24), (1, 17, 33, 1024, 128, 32, 32),
    (2, 1, 1, 32, 1024, 8, 64), (1, 24, 40, 512, 512, 32, 32), (1, 16, 16, 256, 256, 32, 16),
    (2, 13, 21, 64, 256, 32, 32), (1, 9, 20, 64, 768, 16, 48),
    # more than 256 tiles per sample (the statistics merge folds two or more
    # tiles per thread): 288 tiles over 288 workgroups of 256 output channels,
    # and 512 tiles of 128 output channels
    (1, 144, 256, 64, 256, 32, 32), (1, 256, 256, 32, 128, 8, 32),
    # output groups of 2 and of 64 channels (the cases above take 4, 8 and
    # 16, the seeded random problems 1 and 32: every group width the
    # statistics epilogue handles)
    (1, 12, 20, 64, 128, 16, 64), (2, 10, 18, 32, 256, 8, 4),
]


@pytest.mark.parametrize("N,H,W,Ci,Co,G,G2", SHAPES)
def test_plain_conv(gn, dev, oracle, N, H, W, Ci, Co, G, G2):
    print("case plain N=%d H=%d W=%d Ci=%d Co=%d" % (N, H, W, Ci, Co), flush=True)
    x, _, _, wb, bias, _ = make_problem(N, H, W, Ci, Co, seed=100 + Ci + H)
    z, _, _ = run_gpu(gn, dev, N, H, W, Ci, Co, x, None, None, wb, bias, None, G, False, False,
                      None)
    ref, mag = oracle.conv3x3(x, wb, bias, N, H, W, Ci, Co, return_abs=True)
    compare(z, ref, tolerance(ref, mag, Ci, False), "plain conv")


@pytest.mark.parametrize("N,H,W,Ci,Co,G,G2", SHAPES)
def test_gn_silu_conv_with_statistics(gn, dev, oracle, N, H, W, Ci, Co, G, G2):
    print("case gn+silu+conv+stats N=%d H=%d W=%d Ci=%d Co=%d G=%d G2=%d" % (
        N, H, W, Ci, Co, G, G2), flush=True)
    x, gamma, beta, wb, bias, _ = make_problem(N, H, W, Ci, Co, seed=200 + Ci + W)
    z, m2, r2 = run_gpu(gn, dev, N, H, W, Ci, Co, x, gamma, beta, wb, bias, None, G, True, True,
                        G2)
    ref, mag, _, _ = oracle.gn_silu_conv3x3(x, gamma, beta, G, 1e-6, True, wb, bias, N, H, W,
                                            Ci, Co)
    tol = tolerance(ref, mag, Ci, True)
    compare(z, ref, tol, "gn+silu+conv")
    check_stats(m2, r2, ref, tol, N, H * W, Co, G2, 1e-6, "gn+silu+conv")


@pytest.mark.parametrize("N,H,W,Ci,Co,G,G2", [SHAPES[1], SHAPES[4], SHAPES[7], SHAPES[9]])
def test_gn_conv_residual_without_silu(gn, dev, oracle, N, H, W, Ci, Co, G, G2):
    x, gamma, beta, wb, bias, r = make_problem(N, H, W, Ci, Co, seed=300 + Co, res=True)
    z, m2, r2 = run_gpu(gn, dev, N, H, W, Ci, Co, x, gamma, beta, wb, bias, r, G, False, True,
                        G2)
    ref, mag, _, _ = oracle.gn_silu_conv3x3(x, gamma, beta, G, 1e-6, False, wb, bias, N, H, W,
                                            Ci, Co, res=r)
    tol = tolerance(ref, mag, Ci, True)
    compare(z, ref, tol, "gn+conv+residual")
    check_stats(m2, r2, ref, tol, N, H * W, Co, G2, 1e-6, "gn+conv+residual")


def test_silu_without_norm(gn, dev, oracle):
    """apply_silu with no statistics: y = SiLU(x)."""
    N, H, W, Ci, Co = 1, 9, 20, 64, 128
    x, _, _, wb, bias, _ = make_problem(N, H, W, Ci, Co, seed=400)
    z, _, _ = run_gpu(gn, dev, N, H, W, Ci, Co, x, None, None, wb, bias, None, 1, True, False,
                      None)
    xv = oracle.widen(x)
    y = xv / (1.0 + np.exp(-xv))
    ref, mag = oracle.conv3x3(y, wb, bias, N, H, W, Ci, Co, return_abs=True)
    compare(z, ref, tolerance(ref, mag, Ci, True), "silu+conv")


def test_cancellation_stress_statistics(gn, dev, oracle):
    """Output channels far from zero against a small spread: the tile
    moments are centred before they are merged."""
    N, H, W, Ci, Co, G, G2 = 1, 40, 48, 64, 128, 16, 32
    x, gamma, beta, wb, bias, _ = make_problem(N, H, W, Ci, Co, seed=500)
    bias = (bias + 50.0).astype(np.float32)
    wb_small = wb.copy()
    z, m2, r2 = run_gpu(gn, dev, N, H, W, Ci, Co, x, gamma, beta, wb_small, bias, None, G, True,
                        True, G2)
    ref, mag, _, _ = oracle.gn_silu_conv3x3(x, gamma, beta, G, 1e-6, True, wb_small, bias, N, H,
                                            W, Ci, Co)
    tol = tolerance(ref, mag, Ci, True)
    compare(z, ref, tol, "offset outputs")
    check_stats(m2, r2, ref, tol, N, H * W, Co, G2, 1e-6, "offset outputs")


def test_deterministic(gn, dev):
    N, H, W, Ci, Co, G, G2 = 2, 19, 35, 128, 256, 32, 32
    x, gamma, beta, wb, bias, r = make_problem(N, H, W, Ci, Co, seed=600, res=True)
    outs = [run_gpu(gn, dev, N, H, W, Ci, Co, x, gamma, beta, wb, bias, r, G, True, True, G2)
            for _ in range(3)]
    for z, m2, r2 in outs[1:]:
        assert np.array_equal(z, outs[0][0])
        assert np.array_equal(m2, outs[0][1]) and np.array_equal(r2, outs[0][2])


def test_packed_weights_give_the_same_output(gn, dev):
    """Packing once (gn_conv3x3_pack_weights) and calling the packed entry
    gives the unpacked entry's output bit for bit."""
    N, H, W, Ci, Co, G, G2 = 1, 21, 37, 96, 256, 32, 32
    x, gamma, beta, wb, bias, r = make_problem(N, H, W, Ci, Co, seed=650, res=True)
    xd = bits_dev(x, (N, H, W, Ci), dev).permute(0, 3, 1, 2)
    wd = bits_dev(wb, (Co, 3, 3, Ci), dev).permute(0, 3, 1, 2)
    bd = torch.from_numpy(bias).to(dev)
    rd = bits_dev(r, (N, H, W, Co), dev).permute(0, 3, 1, 2)
    with torch.no_grad():
        mean, rstd = gn.group_stats_rows(xd.permute(0, 2, 3, 1).reshape(N, H * W, Ci), G, 1e-6)
        nrm = (mean, rstd, torch.from_numpy(gamma).to(dev), torch.from_numpy(beta).to(dev))
        pw = gn.pack_conv3x3_weight(wd)
        assert pw is not None
        a = gn.conv3x3(xd, wd, bd, norm=nrm, apply_silu=True, residual=rd, next_groups=G2)
        b = gn.conv3x3(xd, pw, bd, norm=nrm, apply_silu=True, residual=rd, next_groups=G2)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_resnet_block_in_a_hip_graph(gn, dev):
    """The fused ResnetBlock2D sequence (statistics, conv1 with GroupNorm+SiLU
    and output statistics, conv2 with GroupNorm+SiLU and the shortcut)
    captured into a HIP graph: every replay, with eager work of the same
    library between replays, equals the eager result bit for bit."""
    N, H, W, C, G = 1, 24, 40, 128, 32
    x, gamma, beta, wb, bias, _ = make_problem(N, H, W, C, C, seed=800)
    xd = bits_dev(x, (N, H, W, C), dev).permute(0, 3, 1, 2)
    wd = bits_dev(wb, (C, 3, 3, C), dev).permute(0, 3, 1, 2)
    bd = torch.from_numpy(bias).to(dev)
    ga = torch.from_numpy(gamma).to(dev)
    be = torch.from_numpy(beta).to(dev)
    rows = xd.permute(0, 2, 3, 1).reshape(N, H * W, C)
    stream = torch.cuda.Stream(dev)

    def block():
        m1, r1 = gn.group_stats_rows(rows, G, 1e-6)
        h, m2, r2 = gn.conv3x3(xd, pw, bd, norm=(m1, r1, ga, be), apply_silu=True, next_groups=G)
        return gn.conv3x3(h, pw, bd, norm=(m2, r2, ga, be), apply_silu=True, residual=xd)

    with torch.no_grad():
        pw = gn.pack_conv3x3_weight(wd)
        with torch.cuda.stream(stream):
            ref = block().clone()
            for _ in range(2):
                block()
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            out = block()
        for rep in range(4):
            with torch.cuda.stream(stream):
                g.replay()
            stream.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "replay %d" % rep
            with torch.cuda.stream(stream):
                other = block()          # eager work between replays
            stream.synchronize()
            assert torch.equal(other.view(torch.int16), ref.view(torch.int16))


def test_unsupported_and_invalid(gn, dev):
    x = torch.zeros(1, 48, 8, 8, device=dev, dtype=torch.bfloat16).to(
        memory_format=torch.channels_last)
    w = torch.zeros(128, 48, 3, 3, device=dev, dtype=torch.bfloat16).to(
        memory_format=torch.channels_last)
    with torch.no_grad():
        assert gn.conv3x3(x, w) is None                                   # Ci % 32
        x2 = torch.zeros(1, 64, 8, 8, device=dev, dtype=torch.bfloat16).to(
            memory_format=torch.channels_last)
        w2 = torch.zeros(128, 64, 3, 3, device=dev, dtype=torch.bfloat16)
        assert gn.conv3x3(x2, w2) is None                                 # weight not CL
        assert gn.conv3x3(x2.contiguous(), w2.to(memory_format=torch.channels_last)) is None
        with pytest.raises(ValueError):
            gn.conv3x3(x2, w2.to(memory_format=torch.channels_last), next_groups=3)


@pytest.mark.parametrize("Ci,Co,H,W", [(512, 512, 128, 128), (256, 256, 256, 256),
                                       (128, 128, 512, 512)])
def test_decoder_size_full(gn, dev, oracle, Ci, Co, H, W):
    """ResnetBlock2D convolutions of the decoder at full size, in the launch
    configuration the benchmark times (128, 512 and 2048 output tiles per
    sample, so the statistics merge folds up to eight tiles per thread):
    GroupNorm+SiLU prologue, residual, every output against the fp64 oracle,
    and the fp32 output statistics against the oracle's fp64 statistics of
    its own output."""
    N, G, G2 = 1, 32, 32
    print("case decoder conv (1,%d,%d,%d) -> %d" % (Ci, H, W, Co), flush=True)
    x, gamma, beta, wb, bias, r = make_problem(N, H, W, Ci, Co, seed=700 + Ci, res=True)
    z, m2, r2 = run_gpu(gn, dev, N, H, W, Ci, Co, x, gamma, beta, wb, bias, r, G, True, True, G2)
    ref, mag, _, _ = oracle.gn_silu_conv3x3(x, gamma, beta, G, 1e-6, True, wb, bias, N, H, W,
                                            Ci, Co, res=r)
    tol = tolerance(ref, mag, Ci, True)
    del mag
    compare(z, ref, tol, "decoder conv")
    check_stats(m2, r2, ref, tol, N, H * W, Co, G2, 1e-6, "decoder conv")

"""Host-side proof that the fused conv kernel's accesses stay in bounds.

gn_conv3x3_plan gives the launch shape; the kernel's index arithmetic is
replayed here with its tile constants (8 x 16 output pixels; 256 lanes as
2 x 2 waves of 64 pixels x 64 channels, or as 1 x 4 waves of 128 pixels x 64
channels when Co is a multiple of 256; chunks of 32 input channels, two LDS
halo buffers with rows of 40 bf16, epilogue rows of 72 fp32): the workgroup
-> (tile, channel block) map
covers every pair once, the halo, weight-fragment, residual and output
addresses stay inside their tensors, every LDS index stays inside its array,
and the statistics partials stay inside their buffer.  The epilogue's
statistics reduction (lane sums, butterflies over the lanes of a wave, the
four waves' sums) is replayed too: every (pixel, channel) of a group is
counted once in that group's sum.
"""
import numpy as np
import pytest

gn = pytest.importorskip("groupnorm_silu_normalization_amd")

TH, TW, BN, BK, KS, OS = 8, 16, 128, 32, 40, 72
HH, HWD = TH + 2, TW + 2
A_ELEMS = HH * HWD * KS
PACK_STEP = 2 * 2 * 2 * 64 * 8             # packed weights per (block, step)
LDS_MAIN = 2 * A_ELEMS                      # bf16 elements: two halo buffers
LDS_EPI_FLOATS = TH * TW * OS

SHAPES = [  # N, H, W, Ci, Co, G2
    (1, 8, 16, 32, 128, 32), (2, 13, 21, 64, 128, 32), (1, 32, 48, 128, 256, 32),
    (1, 5, 7, 32, 128, 8), (1, 64, 64, 512, 512, 32), (3, 9, 17, 96, 384, 24),
    (1, 128, 128, 512, 512, 32), (2, 1, 1, 32, 1024, 64), (1, 17, 33, 1024, 128, 32),
    (1, 9, 20, 64, 768, 48), (2, 7, 40, 32, 256, 16),
    (1, 144, 256, 64, 256, 32), (1, 256, 256, 32, 128, 32),
]


def test_oracle_checked_shapes_reach_the_multi_tile_merge():
    """The GPU parity shapes with more than 256 tiles per sample: the
    statistics merge then folds two or more tiles in some threads, and
    (1, 144, 256) with 256 output channels launches more than 256 workgroups,
    so it runs the two-waves-per-SIMD build of the 128-pixel waves."""
    p = gn.conv_plan(1, 144, 256, 64, 256, 32)
    assert p["tiles_h"] * p["tiles_w"] == 288 and p["wn"] == 4 and p["blocks"] == 288
    q = gn.conv_plan(1, 256, 256, 32, 128, 32)
    assert q["tiles_h"] * q["tiles_w"] == 512 and q["wn"] == 2


def block_map(p, b):
    if p["xcd_map"]:
        xcd, j = b % 8, b // 8
        reps = 8 // p["nb"]
        tile, cb = j * reps + xcd // p["nb"], xcd % p["nb"]
        return (tile, cb) if tile < p["blocks"] // p["nb"] else None
    return (b // p["nb"], b % p["nb"]) if b < p["blocks"] else None


@pytest.mark.parametrize("N,H,W,Ci,Co,G2", SHAPES)
def test_conv_plan_and_indices_in_bounds(N, H, W, Ci, Co, G2):
    p = gn.conv_plan(N, H, W, Ci, Co, G2)
    assert p is not None
    WN = p["wn"]
    assert WN == (4 if Co % 256 == 0 else 2)
    WM = 4 // WN                                 # waves along the pixels
    MI = 4 // WM                                 # 32-pixel blocks per wave
    NT, BNW = 64 * WM * WN, 64 * WN              # lanes, output channels per workgroup
    assert NT == 256
    assert p["tiles_h"] == -(-H // TH) and p["tiles_w"] == -(-W // TW) and p["nb"] == Co // BNW
    tps = p["tiles_h"] * p["tiles_w"]
    assert p["blocks"] == N * tps * p["nb"] and p["grid"] < 2 ** 31
    assert p["xcd_map"] == (8 % p["nb"] == 0)
    if p["xcd_map"]:
        assert p["grid"] % 8 == 0
    seen = set()
    for b in range(p["grid"]):
        m = block_map(p, b)
        if m is not None:
            assert m not in seen
            seen.add(m)
    assert len(seen) == p["blocks"], "every (tile, channel block) runs exactly once"
    # halo pieces: 180 pixels x 4 pieces of 8 channels, PP per lane, clamped
    # to the last piece
    PP = -(-720 // NT)
    v = np.minimum(np.arange(NT)[:, None] + NT * np.arange(PP)[None, :], 719)
    pix, q = v // 4, v % 4
    assert np.all(pix * KS + 8 * q + 8 <= A_ELEMS)
    assert set(v.ravel().tolist()) == set(range(720)), "every halo piece is written"
    # halo fragment reads: wave (wm, wn), block mi, lane -> halo pixel, k offset,
    # in either halo buffer
    lane = np.arange(64)
    fp, fk = lane % 32, 8 * (lane // 32)
    for buf in (0, 1):
        for wm in range(WM):
            for mi in range(MI):
                for kh in range(3):
                    for kw in range(3):
                        hp = (wm * 2 * MI + mi * 2 + fp // 16 + kh) * HWD + fp % 16 + kw
                        assert np.all(buf * A_ELEMS + hp * KS + 16 + fk + 8 <= LDS_MAIN)
                        assert np.all(hp < HH * HWD)
    # packed weight fragments, read from global memory: block cb, step s,
    # k-step ks, wave column wn, block column ni, lane -> 8 bf16 at
    # (cb*nsteps + s)*4096 + ((ks*2 + wn)*2 + ni)*512 + lane*8
    nsteps = Ci // BK * 9
    for cb in (0, Co // BNW - 1):
        for wn in range(WN):
            blk = cb * BNW // BN + wn // 2           # 128-channel packed block
            for ni in (0, 1):
                for step in (0, 1, nsteps - 1):
                    for ks in (0, 1):
                        off = (blk * nsteps + step) * PACK_STEP \
                            + ((ks * 2 + wn % 2) * 2 + ni) * 512 + lane * 8
                        assert off.min() >= 0 and (off + 8).max() <= Co * 9 * Ci
    # the packing kernel's map is a bijection from packed pieces onto the
    # weight tensor's 16-byte pieces
    if Co * 9 * Ci <= 128 * 9 * 1024:
        v = np.arange(Co * 9 * Ci // 8)
        lane_, r = v % 64, v // 64
        ni_, r = r % 2, r // 2
        wn_, r = r % 2, r // 2
        ks_, r = r % 2, r // 2
        step_, cb_ = r % nsteps, r // nsteps
        k_, t_ = step_ // 9, step_ % 9
        co = cb_ * BN + wn_ * 64 + ni_ * 32 + lane_ % 32
        ci = k_ * BK + ks_ * 16 + 8 * (lane_ // 32)
        src = (co * 9 + t_) * Ci + ci
        assert src.min() >= 0 and (src + 8).max() <= Co * 9 * Ci
        assert np.array_equal(np.sort(src // 8), np.arange(Co * 9 * Ci // 8))
    # epilogue staging and the statistics scratch in the same LDS
    r = np.arange(16)
    m = 8 * (r[:, None] // 4) + 4 * (lane[None, :] // 32) + r[:, None] % 4
    pixl = 32 * MI * (WM - 1) + 32 * (MI - 1) + m
    assert (pixl * OS + 63).max() < LDS_EPI_FLOATS and m.max() < 32
    ROWS = NT // 8
    assert (TH * TW) % ROWS == 0
    # statistics LDS: [sums, squares][4 waves][64 channels], 16-byte writes
    tid = np.arange(NT)
    st = (tid >> 6) * 64 + 8 * (tid & 7)
    assert (st + 256 + 8).max() <= 512
    assert max(LDS_MAIN * 2, LDS_EPI_FLOATS * 4) + 512 * 4 + 2 * 1024 * 4 <= 64 * 1024
    # output / residual pieces of valid pixels, statistics partials
    for tile in (0, N * tps - 1):
        n, tin = tile // tps, tile % tps
        h0, w0 = (tin // p["tiles_w"]) * TH, (tin % p["tiles_w"]) * TW
        for pixt in range(TH * TW):
            oh, ow = h0 + pixt // TW, w0 + pixt % TW
            if oh < H and ow < W:
                off = ((n * H + oh) * W + ow) * Co + (Co - BNW) + 64 * (WN - 1) + 8 * 7
                assert off + 8 <= N * H * W * Co
        if G2:
            Cg2 = Co // G2
            assert 64 % Cg2 == 0
            g2 = (Co - 64) // Cg2 + 64 // Cg2 - 1
            assert ((n * tps + tin) * G2 + g2) * 4 + 4 <= N * tps * G2 * 4


def test_conv_plan_declines():
    assert gn.conv_plan(1, 8, 8, 48, 128) is None            # Ci not a multiple of 32
    assert gn.conv_plan(1, 8, 8, 64, 192) is None            # Co not a multiple of 128
    assert gn.conv_plan(1, 8, 8, 2048, 128) is None          # Ci above 1024
    assert gn.conv_plan(1, 8, 8, 64, 512, 4) is None         # groups of 128 channels
    with pytest.raises(ValueError):
        gn.conv_plan(1, 8, 8, 64, 128, 3)                    # Co % G2 != 0
    assert gn.conv_plan(0, 8, 8, 64, 128)["grid"] == 0       # empty: nothing launched
    assert gn.conv_plan(1, 2048, 2048, 512, 128) is None      # sample of 2^31 elements
    assert gn.conv_plan(1, 2048, 1024, 512, 128) is not None  # 2^30: 32-bit offsets hold


def conv_stats_replay(Cg2):
    """The statistics reduction of one 64-channel pass, as bit sets of the
    (pixel, channel) values each sum holds: lane tid (piece q = tid % 8, row
    prow = tid / 8, wave tid / 64) starts with pixels prow + 32 i of channels
    8q + e; the in-lane pairs (Cg2 < 8) or the lane's whole piece (Cg2 >= 8);
    the xor butterfly over lane bits 3-5 and, for Cg2 > 8, over bits 0-2; the
    wave's first row publishes [wave][8q + e]; the sum of a channel is the four
    waves' entries.  No value may be added twice, and each channel's sum must
    hold exactly its group's 128 pixels x Cg2 channels."""
    NT, PIX, ROWS = 256, 4, 32

    def bit(pix, ch):
        return 1 << (pix * 64 + ch)

    def add(a, b):
        assert a & b == 0, "a value counted twice"
        return a | b

    t = [[0] * 8 for _ in range(NT)]
    for tid in range(NT):
        q, prow = tid & 7, tid >> 3
        for e in range(8):
            for i in range(PIX):
                t[tid][e] |= bit(prow + ROWS * i, 8 * q + e)
    if Cg2 >= 8:
        v = []
        for tid in range(NT):
            x = t[tid]
            v.append(add(add(add(x[0], x[1]), add(x[2], x[3])), add(add(x[4], x[5]), add(x[6], x[7]))))
        masks = [8, 16, 32] + [m for m in (1, 2, 4) if 8 * m < Cg2]
        for m in masks:
            v = [add(v[tid], v[tid ^ m]) for tid in range(NT)]
        t = [[v[tid]] * 8 for tid in range(NT)]
    else:
        for tid in range(NT):
            x = t[tid]
            if Cg2 >= 2:
                for e in range(0, 8, 2):
                    x[e] = x[e + 1] = add(x[e], x[e + 1])
            if Cg2 >= 4:
                for h in (0, 4):
                    for e in (h, h + 1):
                        x[e] = x[e + 2] = add(x[e], x[e + 2])
        for m in (8, 16, 32):
            t = [[add(t[tid][e], t[tid ^ m][e]) for e in range(8)] for tid in range(NT)]
    st = {}
    for tid in range(NT):
        if tid & 63 < 8:
            for e in range(8):
                idx = (tid >> 6) * 64 + 8 * (tid & 7) + e
                assert idx < 256 and idx not in st
                st[idx] = t[tid][e]
    for c in range(64):
        total = 0
        for w in range(4):
            total = add(total, st[w * 64 + c])
        g0 = c // Cg2 * Cg2
        want = 0
        for pix in range(128):
            for ch in range(g0, g0 + Cg2):
                want |= bit(pix, ch)
        assert total == want, (Cg2, c)


@pytest.mark.parametrize("Cg2", [1, 2, 4, 8, 16, 32, 64])
def test_conv_stats_reduction_counts_each_value_once(Cg2):
    conv_stats_replay(Cg2)

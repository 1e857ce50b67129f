"""Host-side proof that every kernel access stays in bounds, on the CPU.

For each shape the library's own launch plan (gn_plan_rows_dtype) is read
back, and the kernels' index arithmetic is replayed here: the lane->element
slot map of a tile, the element range each workgroup of the statistics and
apply passes touches, the partial tile at the end of a sample, the pivot
reads, the partial-sum slots, the LDS slots of the workgroup reduction and
the grid sizes.  It also checks that the chunks tile each sample exactly
once, so no element is skipped or counted twice, and that every slot of a
lane holds one fixed channel.
"""
from math import gcd

import numpy as np
import pytest

gn = pytest.importorskip("groupnorm_silu_normalization_amd")

THREADS = 256
FINALIZE_BATCH = 16   # partials per thread per batch in the fused finalize
BF16, F16, F32 = 0, 1, 2
WIDE = {BF16: 8, F16: 8, F32: 4}   # elements per 16-byte access

SHAPES = [
    # the five decoder shapes (N, L, C, G)
    (1, 64 * 64, 128, 32), (1, 128 * 128, 512, 32), (1, 512 * 512, 512, 32),
    (1, 1024 * 1024, 256, 32), (1, 1024 * 1024, 128, 32),
    # rows case, ragged tails, small and extreme power-of-two channel counts
    (1, 16384, 512, 32), (3, 70001, 128, 32), (2, 5000, 64, 8), (2, 1, 8, 8),
    (1, 1, 1, 1), (1, 3, 2, 1), (2, 7, 4, 2), (4, 5, 2, 2), (1, 257, 2048, 2048),
    (1, 257, 2048, 1), (2, 129, 1024, 512), (2, 33, 512, 256), (7, 3, 16, 4),
    (64, 100, 32, 32), (1, 2 ** 22, 512, 32), (2 ** 12, 1, 8, 1), (1, 9999, 1, 1),
    (2, 131072, 64, 8), (5, 6, 4, 4),
]
# channel counts that are not powers of two, or above 2048 (UNet widths and
# their concatenations, odd and prime counts, ragged row counts)
WIDE_SHAPES = [
    (2, 4096, 320, 32), (1, 1024, 640, 32), (2, 257, 960, 32), (1, 4097, 1280, 32),
    (1, 999, 1920, 32), (2, 513, 2560, 32), (1, 129, 4096, 32), (1, 65, 8192, 32),
    (3, 77, 96, 32), (2, 33, 24, 8), (1, 5, 3, 1), (2, 7, 3, 3), (1, 11, 5, 5),
    (4, 9, 300, 30), (1, 1, 300, 300), (2, 17, 250, 10), (1, 1000, 6144, 32),
    (1, 100, 1536, 48), (2, 31, 768, 24), (1, 1, 2560, 2560), (2, 3, 1000, 1000),
]
DTYPES = (BF16, F16, F32)


def lane_offsets(p):
    """o[tid, j] for the active lanes."""
    A, W, S = p["A"], p["W"], p["slots"]
    tid = np.arange(A)[:, None]
    j = np.arange(S)[None, :]
    return ((j // W) * A + tid) * W + j % W


def check_layout(p, E, C, dtype):
    A, W, S, T = p["A"], p["W"], p["slots"], p["T"]
    NV = S // W
    assert W in (1, WIDE[dtype]) and S % W == 0 and NV in (1, 2, 4)
    assert W == 1 or (dtype == F32 and NV >= 2) or dtype != F32
    assert E % W == 0, "a 16-byte access must not straddle two samples"
    assert 0 < A <= p["threads"] and T == A * S
    assert T % C == 0, "a tile must be whole rows so each slot keeps one channel"
    # the kernels take masks and shifts for channel and group indices when all
    # 256 lanes are busy: that must happen exactly for power-of-two C
    assert (A == THREADS) == (C & (C - 1) == 0)
    o = lane_offsets(p)
    # the slot map is a permutation of the tile
    assert np.array_equal(np.sort(o.ravel()), np.arange(T))
    # each access of W slots is contiguous and W-aligned; one wave instruction
    # (64 lanes, same access) covers 64*W contiguous elements
    for a in range(NV):
        blk = o[:, a * W:(a + 1) * W]
        assert np.all(blk[:, 0] % W == 0)
        assert np.all(np.diff(blk, axis=1) == 1)
        for w0 in range(0, A, 64):
            starts = blk[w0:w0 + 64, 0]
            assert np.array_equal(starts, starts[0] + W * np.arange(starts.size))
    return o


def chunks(tiles, full, tpc, K, rem=0):
    """Chunk k: tiles [k*tpc + min(k, rem), + tpc + (k < rem)), clipped to the
    sample (step 1: rem = 0; step 3: an even split, rem = tiles % K)."""
    out = []
    for k in range(K):
        t_begin = k * tpc + min(k, rem)
        t_end = min(t_begin + tpc + (1 if k < rem else 0), tiles)
        out.append((t_begin, t_end, max(min(t_end, full), t_begin)))
    return out


def wide_layout(E, C, dtype, nbytes):
    """(W, NV, 320) when both passes take 320-lane workgroups: a tensor above
    16 MiB whose 256-lane layout leaves a quarter or more of the lanes idle or
    needs more than the minimal accesses, and 320 lanes are all busy with the
    minimal ones; else None."""
    base = expected_layout(E, C, dtype)
    if base is None or nbytes <= 16 << 20:
        return None
    W, nv, A = base
    nv_min = 2 if W == 4 else 1
    if W == 1 or (nv == nv_min and 4 * A >= 3 * THREADS):
        return None
    m = C // gcd(C, W * nv_min)
    return (W, nv_min, 320) if 320 % m == 0 else None


def check_streaming_pass(N, E, p, o, tpc, K, rem=0):
    T, tiles, full = p["T"], p["tiles"], p["full"]
    assert N * K < 2 ** 24, "grid too large"
    assert tiles == -(-E // T) and full == E // T
    cs = chunks(tiles, full, tpc, K, rem)
    # the chunks cover tiles [0, tiles) once, in order
    assert cs[0][0] == 0 and cs[-1][1] == tiles
    for a, b in zip(cs, cs[1:]):
        assert a[1] == b[0] and a[0] < a[1]
    for t_begin, t_end, t_full_end in cs:
        assert t_begin < tiles
        assert t_full_end * T <= E                   # whole tiles inside the sample
        if t_end > t_full_end:                       # the partial last tile
            assert t_end == t_full_end + 1 == tiles
            offs = t_full_end * T + o.ravel()
            live = offs[offs < E]
            # the in-bounds slots are exactly the tail elements, once each
            assert np.array_equal(np.sort(live), np.arange(t_full_end * T, E))


def check_lds(p, C, G):
    """The workgroup reduction of step 1: slot (tid, j) goes to LDS entry
    o(tid, j) < T <= lanes*slots (the LDS arrays); group g's P = T/G entries
    are read back by the first 256 threads (every workgroup width)."""
    T, S = p["T"], p["slots"]
    Cg = C // G
    P = T // G
    assert T <= p["threads"] * S
    seen = np.zeros(T, np.int64)
    if G <= THREADS:
        tg = THREADS // G
        per = -(-P // tg)
        for g in range(G):
            for part in range(tg):
                for e in range(part * per, min(P, (part + 1) * per)):
                    i = (e // Cg) * C + g * Cg + e % Cg
                    assert 0 <= i < T and (i % C) // Cg == g
                    seen[i] += 1
        # the tree over the tg parts of group g stays inside [g*tg, g*tg + tg)
        assert G * tg <= THREADS
    else:
        for g in range(G):
            for e in range(P):
                i = (e // Cg) * C + g * Cg + e % Cg
                assert 0 <= i < T and (i % C) // Cg == g
                seen[i] += 1
    assert np.all(seen == 1), "each LDS slot is summed into exactly one group once"


def check_plan(N, L, C, G, dtype):
    p = gn.plan_rows(N, L, C, G, dtype)
    assert p is not None, (N, L, C, G, dtype)
    E = L * C
    wide = wide_layout(E, C, dtype, N * E * (4 if dtype == F32 else 2))
    want = wide or expected_layout(E, C, dtype)
    assert (p["W"], p["slots"] // p["W"], p["A"]) == want, (N, L, C, G, dtype, p)
    assert p["threads"] == (320 if wide else THREADS)
    o = check_layout(p, E, C, dtype)
    check_streaming_pass(N, E, p, o, p["tpc1"], p["K1"])
    # step 3: K2 chunks splitting the tiles evenly, K2 from whole rounds of 256
    assert p["tpc2"] == p["tiles"] // p["K2"] >= 1
    check_streaming_pass(N, E, p, o, p["tpc2"], p["K2"], p["tiles"] % p["K2"])
    # each lane slot keeps one channel across tiles: o mod C, and its group
    ch = o % C
    assert np.all((ch // (C // G)) < G)
    # pivot reads x[n, 0, g*Cg] lie in row 0 of the sample
    assert (G - 1) * (C // G) < E
    # partial-sum slots (n*K1 + k)*G + g, written by step 1 and read by the
    # finalize (fused tail: thread g + G*j, j < 256//G, reads k = j, j + 256//G, ...)
    nparts = N * G * p["K1"]
    assert ((N - 1) * p["K1"] + p["K1"] - 1) * G + G - 1 < nparts
    pad = (FINALIZE_BATCH - 1) * THREADS   # finalize over-read padding after the squares
    if G <= THREADS:
        tpg = THREADS // G
        assert tpg * G <= THREADS
        seen = sorted(k for j in range(tpg) for k in range(j, p["K1"], tpg))
        assert seen == list(range(p["K1"]))
        # a fused-finalize batch loads slots kk + b*tpg, b < FINALIZE_BATCH, for
        # every kk = j + m*FINALIZE_BATCH*tpg < K1, adding only those < K1: the
        # highest float it reads, relative to the start of the partial squares
        # of the last sample, stays inside the squares and the padding
        K = p["K1"]
        kk_last = max(kk for j in range(tpg) for kk in range(j, K, FINALIZE_BATCH * tpg))
        top = ((N - 1) * K + kk_last + (FINALIZE_BATCH - 1) * tpg) * G + G - 1
        assert top < nparts + pad
        # the late finalize: a thread with no part (j >= K1, or a thread past
        # tpg*G) loads part 0's batch and adds none of it -- no higher
        top0 = ((N - 1) * K + (FINALIZE_BATCH - 1) * tpg) * G + G - 1
        assert top0 <= top
    # arrival counters: one word per sample, or a two-level count of 8 groups
    # plus a total, each on its own 128-byte line, when a sample has >= 64 chunks
    words = N * ((8 + 1) * 32 if p["K1"] >= 64 else 1)
    counters = -(-4 * words // 256) * 256
    single = gn.plan_single_launch(N, L, C, G, dtype)["single_launch"]
    # the single launch keeps everything on chip (the three-step plan above
    # still serves steps 1-2 and 3 called alone)
    assert p["scratch_bytes"] == (0 if single else
                                  counters + 4 * (2 * nparts + pad + 2 * N * G))
    assert N * G < 2 ** 24
    check_lds(p, C, G)
    # step 1's plain-load tail: the whole chunk when the tensor fits the
    # 256 MiB cache, else the chunk's share of one cache's worth (at least 1)
    nbytes = N * E * (4 if dtype == F32 else 2)
    cache = 256 << 20
    want = p["tpc1"] if nbytes <= cache else max(1, -(-p["tpc1"] * cache // nbytes))
    assert p["stats_plain_tail"] == want
    # the late finalize (step 2 in every step-3 workgroup): small x, G <= 256,
    # and one finalize batch per thread covering the sample's chunks, so its
    # partial reads are exactly the fused finalize's first batch (bounded above)
    late = (G <= THREADS and nbytes <= 16 << 20
            and p["K1"] <= FINALIZE_BATCH * (THREADS // G))
    assert p["late_finalize"] == int(late)
    return p


@pytest.mark.parametrize("N,L,C,G", SHAPES)
def test_plan_keeps_every_access_in_bounds(N, L, C, G):
    for dtype in DTYPES:
        check_plan(N, L, C, G, dtype)


@pytest.mark.parametrize("N,L,C,G", WIDE_SHAPES)
def test_wide_plan_keeps_every_access_in_bounds(N, L, C, G):
    for dtype in DTYPES:
        if supported(L * C, C, dtype):
            check_plan(N, L, C, G, dtype)
        else:
            assert gn.plan_rows(N, L, C, G, dtype) is None


def supported(E, C, dtype):
    """The supported set as the header states it."""
    if C > 8192:
        return False
    Wd = WIDE[dtype]
    W = Wd if E % Wd == 0 else 1
    nvs = (2, 4) if W == 4 else (1, 2, 4)
    return any(C // gcd(C, W * nv) <= THREADS for nv in nvs)


def test_power_of_two_layout_is_the_2048_element_tile():
    # 16-bit types: one 16-byte access per lane; fp32: two; every lane busy
    for C in (8, 16, 64, 128, 256, 512, 1024, 2048):
        for dtype in DTYPES:
            if dtype == F32 and C > 2048:
                continue
            p = gn.plan_rows(1, 4096, C, 8 if C >= 8 else 1, dtype)
            assert (p["A"], p["T"], p["slots"]) == (256, 2048, 8)
            assert p["W"] == WIDE[dtype]


def expected_layout(E, C, dtype):
    """(W, NV, A) by the plan's rule: the smallest NV with at least half of
    the 256 lanes busy, else the NV with the most busy lanes."""
    Wd = WIDE[dtype]
    W = Wd if E % Wd == 0 else 1
    best = None
    for nv in ((2, 4) if W == 4 else (1, 2, 4)):
        m = C // gcd(C, W * nv)
        if m > THREADS:
            continue
        A = (THREADS // m) * m
        if best is None or A > best[2]:
            best = (W, nv, A)
        if 2 * best[2] >= THREADS:
            break
    return best


def test_wide_layouts_follow_the_rule():
    for C in (320, 640, 960, 1280, 1920, 2560, 4096, 8192, 96, 24, 3, 300, 1000, 6144):
        for L in (1, 8, 4096):
            for dtype in DTYPES:
                nbytes = L * C * (4 if dtype == F32 else 2)
                want = wide_layout(L * C, C, dtype, nbytes) or expected_layout(L * C, C, dtype)
                p = gn.plan_rows(1, L, C, 1, dtype)
                if want is None:
                    assert p is None
                    continue
                assert (p["W"], p["slots"] // p["W"], p["A"]) == want, (C, L, dtype, p)
    # UNet channel counts in bf16 up to 16 MiB: one 16-byte access per lane
    # where half the lanes suffice (1280: 160 lanes), two for 2560 (160 lanes)
    assert [gn.plan_rows(1, 1024, C, 32)["slots"] for C in (320, 1280, 2560, 8192)] == \
        [8, 8, 16, 32]
    assert [gn.plan_rows(1, 1024, C, 32)["A"] for C in (320, 1280, 2560, 8192)] == \
        [240, 160, 160, 256]
    # above 16 MiB, 1280 and 2560 take 320-lane workgroups, one access per lane
    for C in (1280, 2560):
        p = gn.plan_rows(1, 16384, C, 32)
        assert (p["A"], p["slots"], p["T"], p["threads"]) == (320, 8, 2560, 320)
    assert gn.plan_rows(1, 16384, 320, 32)["threads"] == 256
    assert gn.plan_rows(1, 16384, 960, 32)["threads"] == 256


def test_supported_set_matches_the_header_rule():
    Ls = (1, 3, 8, 16)
    for C in list(range(1, 300)) + [320, 640, 960, 1000, 1028, 1280, 1920, 2056, 2560, 3000,
                                    4096, 4100, 5120, 6144, 8192, 8200, 16384]:
        for L in Ls:
            for dtype in DTYPES:
                got = gn.plan_rows(1, L, C, 1, dtype) is not None
                assert got == supported(L * C, C, dtype), (C, L, dtype)
    # every C <= 256, and multiples of 8 up to 2048 in 16-bit types
    assert all(gn.plan_rows(1, 3, C, 1) is not None for C in range(1, 257))
    assert all(gn.plan_rows(1, 8, C, 1) is not None for C in range(8, 2049, 8))
    assert all(gn.plan_rows(1, 8, C, 1, F32) is not None for C in range(4, 1025, 4))


def test_plan_is_shape_only_and_bounded():
    # statistics workgroups stay near the target, so partials stay small
    for N, L, C, G in SHAPES + WIDE_SHAPES:
        p = gn.plan_rows(N, L, C, G)
        if p is None:
            continue
        total = N * p["tiles"]
        assert p["tpc1"] <= 1024                       # each lane's sequential run
        assert N * p["K1"] <= max(256, -(-total // 1024)) + N
        assert N * p["K2"] <= 2048 + N
        assert p == gn.plan_rows(N, L, C, G)
    # the decoder shapes: one statistics workgroup per CU of an MI355X from
    # 64 MiB up; below 16 MiB at most 128 workgroups of at least 8 tiles
    for N, L, C, G in SHAPES[2:5]:
        assert gn.plan_rows(N, L, C, G)["K1"] == 256
    assert gn.plan_rows(*SHAPES[0])["K1"] == 256 // 8        # 256 tiles
    assert gn.plan_rows(*SHAPES[1])["K1"] == 128              # 4096 tiles, 16 MiB
    for N, L, C, G in SHAPES + WIDE_SHAPES:
        p = gn.plan_rows(N, L, C, G)
        if p is None or N * L == 0:
            continue
        blocks = 128 if N * L * C * 2 <= 16 << 20 else 256
        assert N * p["K1"] <= max(blocks, -(-N * p["tiles"] // 1024)) + N
        assert p["tpc1"] >= 8


def test_plan_declines_like_the_entry_points():
    assert gn.plan_rows(1, 16, 257, 1) is None        # prime above 256: no layout
    assert gn.plan_rows(1, 16, 3000, 1) is None       # 8*375: no layout
    assert gn.plan_rows(1, 16, 16384, 32) is None     # C > GN_MAX_CHANNELS
    assert gn.plan_rows(1, 16, 96, 32) is not None    # widened: not a power of two
    assert gn.plan_rows(1, 16, 4096, 32) is not None  # widened: C > 2048
    with pytest.raises(ValueError):
        gn.plan_rows(1, 16, 64, 3)                    # C % G != 0
    assert gn.plan_rows(0, 16, 64, 32)["K1"] == 0     # empty: nothing launched


# ---------------------------------------------------------------- single launch
STRIP_THREADS, STRIP_PIECES = 1024, 2
STRIP_SHAPES = [
    (2, 32 * 32, 256, 32), (1, 256, 128, 32), (4, 2048, 256, 32), (16, 256, 64, 32),
    (3, 999, 64, 32), (2, 77, 8, 8), (1, 5, 16, 1), (4, 1000, 128, 128), (2, 513, 256, 256),
    (1, 1, 8, 1), (5, 123, 16, 16), (1, 1024, 32, 32), (8, 1024, 128, 32), (2, 256, 1024, 32),
    (1, 32, 4096, 8), (1, 16, 2048, 4), (2, 1000, 512, 32), (16, 1024, 128, 32),
    # not taken: too many rows per lane, too many workgroups, too large, odd groups
    (1, 64 * 64, 128, 32), (32, 256, 128, 32), (1, 128 * 128, 512, 32), (2, 1024, 96, 32),
]


def strip_replay(N, L, C, G, dtype):
    """Replays gn_strip's index arithmetic for the plan the library reports:
    every access in bounds, every element of x read (and y written) exactly
    once, each lane's slots on fixed channels of its own strip, and the LDS
    entries of each group covering exactly its channels.  False when the
    shape does not take the single launch."""
    q = gn.plan_single_launch(N, L, C, G, dtype)
    if not q["single_launch"]:
        assert all(v == 0 for v in q.values())
        return False
    es = 4 if dtype == F32 else 2
    W = 16 // es
    Cg = C // G
    gpw, P, blocks, NT = q["groups_per_workgroup"], q["pieces_per_row"], q["workgroups"], q["threads"]
    assert NT == STRIP_THREADS and (C * es) % 16 == 0 and N * L * C * es <= 4 << 20
    assert P & (P - 1) == 0 and 1 <= P <= 64 and gpw * Cg == P * W
    S = G // gpw
    assert blocks == N * S and blocks <= 256
    SUB = min(Cg, W)
    NS = W // SUB
    NW = NT // 64
    rstep = NT // P
    assert q["pieces_per_lane"] == -(-L // rstep) <= STRIP_PIECES
    xcd = blocks % 8 == 0
    seen = np.zeros(N * L * C, dtype=np.int32)
    strips = set()
    tid = np.arange(NT)
    for b0 in range(blocks):
        b = (b0 % 8) * (blocks // 8) + b0 // 8 if xcd else b0
        n, strip = divmod(b, S)
        strips.add((n, strip))
        cs = strip * gpw * Cg
        p = tid & (P - 1)
        r0 = tid // P
        cw = p * W
        for j in range(W):                    # pivots: group starts inside the strip
            assert np.all((cw + j) // Cg < gpw)
        for k in range(STRIP_PIECES):         # pieces: rows r0 + k*rstep < L
            r = r0 + k * rstep
            ok = r < L
            base = n * L * C + cs + r[ok] * C + cw[ok]
            assert np.all(base >= 0) and np.all(base + W <= N * L * C)
            assert np.all((base * es) % 16 == 0)
            for j in range(W):
                seen[base + j] += 1
        ent = (np.arange(NW)[:, None] * P + np.arange(P)[None, :]) * NS
        assert ent.max() + NS - 1 < NW * 64 * NS
        EPW = Cg // W if Cg > W else 1
        EN = EPW * NW
        assert gpw * EN <= NT and EN & (EN - 1) == 0 and gpw <= 64 * NS
        for lg in range(gpw):
            chans = set()
            for e in range(EN):
                w, k = divmod(e, EPW)
                if Cg > W:
                    pc, part = lg * EPW + k, 0
                else:
                    pc, part = (lg * Cg) // W, ((lg * Cg) % W) // SUB
                assert 0 <= pc < P and 0 <= part < NS
                chans |= set(range(pc * W + part * SUB, pc * W + part * SUB + SUB))
            assert chans == set(range(lg * Cg, (lg + 1) * Cg)), "entries of a group"
    assert len(strips) == blocks
    assert np.all(seen == 1), "each element once"
    return True


@pytest.mark.parametrize("N,L,C,G", STRIP_SHAPES)
@pytest.mark.parametrize("dtype", DTYPES)
def test_single_launch_indices_in_bounds(N, L, C, G, dtype):
    if gn.plan_rows(N, L, C, G, dtype) is None:
        pytest.skip("declined")
    strip_replay(N, L, C, G, dtype)


def test_single_launch_selection():
    """The single launch's domain: at most 4 MiB, 16-byte rows, groups that
    fill or split into a power of two of 16-byte pieces, at most 256
    workgroups and two pieces per lane."""
    on = lambda *a: gn.plan_single_launch(*a)["single_launch"] == 1  # noqa: E731
    assert on(2, 1024, 256, 32, BF16) and on(8, 1024, 128, 32, BF16) and on(2, 1024, 256, 32, F32)
    assert on(1, 2048, 128, 32, BF16) and on(16, 1024, 128, 32, BF16)
    assert not on(1, 4096, 128, 32, BF16)          # four pieces per lane
    assert not on(1, 16384, 512, 32, BF16)         # 16 MiB
    assert not on(32, 256, 128, 32, BF16)          # 512 workgroups
    assert not on(16, 256, 256, 32, BF16)          # 512 workgroups
    assert not on(1, 256, 4, 1, BF16)              # 8-byte rows
    assert not on(1, 256, 96, 32, BF16)            # Cg = 3
    assert not on(1, 256, 384, 16, BF16)           # Cg = 24: three pieces
    assert on(1, 256, 384, 48, BF16)               # Cg = 8
    n_on = sum(strip_replay(*s, BF16) for s in STRIP_SHAPES)
    assert n_on == len(STRIP_SHAPES) - 4


def wave_reduction_replay(C, G):
    """The wave-level partial reduction of step 1 (power-of-two 16-byte
    layouts of 16-bit types: 256 lanes, lane tid holding channels
    8*(tid mod C/8) .. +7 of row tid // (C/8); groups of 8 channels or
    more, so a lane's slots lie in one group), replayed with the kernel's
    own index arithmetic on sets of (lane, slot) ids: the butterfly over the
    lane bits that keep the group, one LDS entry per (wave, group) written by
    its leader lane, and thread g adding the entries of the waves whose
    channel blocks meet group g.  Each group's partial must be exactly the
    slots of its channels, each once, and every LDS index in bounds and
    written once."""
    Cg = C // G
    assert Cg >= 8
    cb = C >> 3
    gb = Cg >> 3
    NT, W = 256, 8
    red = {}
    for wave in range(NT // 64):
        masks = [m for m in (1, 2, 4, 8, 16, 32) if m < gb or m >= cb]
        for lane in range(64):
            tid = wave * 64 + lane
            if not ((lane & (gb - 1)) == 0 and (cb >= 64 or lane < cb)):
                continue
            # the leader's sum after the butterfly: every slot of the lanes
            # reachable from it by the masks
            orbit = {lane}
            for m in masks:
                orbit |= {o ^ m for o in orbit}
            idx = wave * G + (tid & (cb - 1)) // gb
            assert 0 <= idx < 4 * G <= NT * W and idx not in red
            red[idx] = [(wave * 64 + o, j) for o in sorted(orbit) for j in range(W)]
    for g in range(G):
        b0, b1 = g * gb, g * gb + gb
        total = []
        for w in range(NT // 64):
            lo = 0 if cb <= 64 else (w * 64) & (cb - 1)
            hi = cb if cb <= 64 else lo + 64
            if b0 < hi and b1 > lo:
                assert w * G + g in red, (C, G, g, w)
                total.extend(red[w * G + g])
        want = [(tid, j) for tid in range(NT) for j in range(W)
                if ((8 * (tid & (cb - 1)) + j) // Cg) == g]
        assert sorted(total) == sorted(want), (C, G, g)


@pytest.mark.parametrize("C", [8, 16, 32, 64, 128, 256, 512, 1024, 2048])
def test_wave_reduction_counts_each_slot_once(C):
    for G in [g for g in (1, 2, 4, 8, 16, 32, 64, 128, 256) if C % g == 0 and C // g >= 8]:
        wave_reduction_replay(C, G)


def narrow_wave_reduction_replay(C, G):
    """The wave-level reduction for groups narrower than a lane's 8 channels
    (Cg = 8 / PER): each lane sums its Cg slots per group, the butterfly runs
    over the row bits of the wave, the first row's lanes write PER entries,
    and thread g adds the entries of the waves holding its channel block."""
    Cg = C // G
    assert Cg < 8 and 8 % Cg == 0
    PER = 8 // Cg
    cb = C >> 3
    NT, W = 256, 8
    red = {}
    for wave in range(NT // 64):
        masks = [m for m in (1, 2, 4, 8, 16, 32) if m >= cb]
        for lane in range(64):
            tid = wave * 64 + lane
            if not (cb >= 64 or lane < cb):
                continue
            orbit = {lane}
            for m in masks:
                orbit |= {o ^ m for o in orbit}
            blk = tid & (cb - 1)
            for h in range(PER):
                idx = wave * G + blk * PER + h
                assert 0 <= idx < 4 * G <= NT * W and idx not in red
                red[idx] = [(wave * 64 + o, h * Cg + u) for o in sorted(orbit) for u in range(Cg)]
    for g in range(G):
        b = g // PER
        total = []
        for w in range(NT // 64):
            lo = 0 if cb <= 64 else (w * 64) & (cb - 1)
            hi = cb if cb <= 64 else lo + 64
            if lo <= b < hi:
                assert w * G + g in red, (C, G, g, w)
                total.extend(red[w * G + g])
        want = [(tid, j) for tid in range(NT) for j in range(W)
                if ((8 * (tid & (cb - 1)) + j) // Cg) == g]
        assert sorted(total) == sorted(want), (C, G, g)


@pytest.mark.parametrize("C", [8, 16, 32, 64, 128, 256])
def test_narrow_wave_reduction_counts_each_slot_once(C):
    for Cg in (1, 2, 4):
        if C % Cg == 0 and C // Cg <= 256:
            narrow_wave_reduction_replay(C, C // Cg)

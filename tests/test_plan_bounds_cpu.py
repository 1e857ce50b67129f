"""Host-side proof that every kernel access stays in bounds, on the CPU.

For each shape the library's own launch plan (gn_plan_rows) is read back, and
the kernels' index arithmetic is replayed here: the element range each
workgroup of the statistics and apply passes touches, the partial tile at the
end of a sample, the pivot reads, the partial-sum slots, the LDS slots of the
workgroup reduction and the grid sizes.  It also checks that the chunks tile
each sample exactly once, so no element is skipped or counted twice.
"""
import numpy as np
import pytest

gn = pytest.importorskip("groupnorm_silu_normalization_amd")

THREADS = 256
SHAPES = [
    # the five decoder shapes (N, L, C, G)
    (1, 64 * 64, 128, 32), (1, 128 * 128, 512, 32), (1, 512 * 512, 512, 32),
    (1, 1024 * 1024, 256, 32), (1, 1024 * 1024, 128, 32),
    # rows case, ragged tails, small and extreme channel counts
    (1, 16384, 512, 32), (3, 70001, 128, 32), (2, 5000, 64, 8), (2, 1, 8, 8),
    (1, 1, 1, 1), (1, 3, 2, 1), (2, 7, 4, 2), (4, 5, 2, 2), (1, 257, 2048, 2048),
    (1, 257, 2048, 1), (2, 129, 1024, 512), (2, 33, 512, 256), (7, 3, 16, 4),
    (64, 100, 32, 32), (1, 2 ** 22, 512, 32), (2 ** 12, 1, 8, 1), (1, 9999, 1, 1),
    (2, 131072, 64, 8), (5, 6, 4, 4),
]


def log2(v):
    return int(v).bit_length() - 1


def chunks(plan_tiles, full, tpc, K):
    out = []
    for k in range(K):
        t_begin = k * tpc
        t_end = min(t_begin + tpc, plan_tiles)
        out.append((t_begin, t_end, min(t_end, full)))
    return out


def check_streaming_pass(N, E, vec, tiles, full, tpc, K):
    TILE = THREADS * vec
    assert N * K < 2 ** 24, "grid too large"
    cs = chunks(tiles, full, tpc, K)
    # the chunks cover tiles [0, tiles) once, in order
    assert cs[0][0] == 0 and cs[-1][1] == tiles
    for a, b in zip(cs, cs[1:]):
        assert a[1] == b[0] and a[0] < a[1]
    for t_begin, t_end, t_full_end in cs:
        assert t_begin < tiles
        if t_full_end > t_begin:
            assert t_full_end * TILE <= E            # whole tiles inside the sample
        if t_end > max(t_full_end, t_begin):         # the partial last tile
            tt = max(t_full_end, t_begin)
            offs = tt * TILE + np.arange(THREADS) * vec
            live = offs[offs < E]
            assert live.size == 0 or live.max() + vec - 1 < E
            covered = live.size * vec
            assert tt * TILE + covered == E          # every tail element read once
    assert full * TILE <= E <= tiles * TILE and tiles == -(-E // TILE)


def lds_slots(C, G, vec):
    TILE = THREADS * vec
    cg_shift = log2(C // G)
    cgm = (1 << cg_shift) - 1
    seen = np.zeros(TILE, np.int64)
    if G <= THREADS:
        tg = THREADS // G
        for tid in range(THREADS):
            g, part = divmod(tid, tg)
            for j in range(vec):
                e = part * vec + j
                i = (e >> cg_shift) * C + (g << cg_shift) + (e & cgm)
                assert 0 <= i < TILE and (i % C) // (C // G) == g
                seen[i] += 1
    else:
        P = TILE // G
        for g in range(G):
            for e in range(P):
                i = (e >> cg_shift) * C + (g << cg_shift) + (e & cgm)
                assert 0 <= i < TILE and (i % C) // (C // G) == g
                seen[i] += 1
    assert np.all(seen == 1), "each LDS slot is summed into exactly one group once"


@pytest.mark.parametrize("N,L,C,G", SHAPES)
def test_plan_keeps_every_access_in_bounds(N, L, C, G):
    p = gn.plan_rows(N, L, C, G)
    assert p is not None
    E = L * C
    vec = p["vec"]
    assert vec in (1, 8) and E % vec == 0
    assert THREADS * vec % C == 0, "a tile must start on a row boundary"
    check_streaming_pass(N, E, vec, p["tiles"], p["full"], p["tpc1"], p["K1"])
    check_streaming_pass(N, E, vec, p["tiles"], p["full"], p["tpc2"], p["K2"])
    # pivot reads x[n, 0, g*Cg] lie in row 0 of the sample
    assert (G - 1) * (C // G) < E
    # partial-sum slots (n*K1 + k)*G + g, written by step 1 and read by the
    # finalize (fused tail: thread g + G*j reads k = j, j + 256/G, ...)
    nparts = N * G * p["K1"]
    assert ((N - 1) * p["K1"] + p["K1"] - 1) * G + G - 1 < nparts
    if G <= THREADS:
        tpg = THREADS // G
        for j in range(tpg):
            ks = range(j, p["K1"], tpg)
            assert all(((N - 1) * p["K1"] + k) * G + (G - 1) < nparts for k in ks)
        # every chunk of every group is read exactly once by the tail
        seen = sorted(k for j in range(tpg) for k in range(j, p["K1"], tpg))
        assert seen == list(range(p["K1"]))
    counters = -(-4 * N // 256) * 256   # one arrival counter per sample
    assert p["scratch_bytes"] == counters + 4 * (2 * nparts + 2 * N * G)
    assert N * G < 2 ** 24
    if C * 8 <= 65536:
        lds_slots(C, G, vec)
    # the reverse walk of the apply pass is a bijection on its workgroups
    nb = N * p["K2"]
    assert sorted(nb - 1 - b for b in range(min(nb, 5000))) == list(range(nb - min(nb, 5000), nb))


def test_plan_is_shape_only_and_bounded():
    # statistics workgroups stay near the target, so partials stay small
    for N, L, C, G in SHAPES:
        p = gn.plan_rows(N, L, C, G)
        total = N * p["tiles"]
        assert p["tpc1"] <= 1024                       # each lane's sequential run
        assert N * p["K1"] <= max(256, -(-total // 1024)) + N
        assert N * p["K2"] <= 2048 + N
        assert p == gn.plan_rows(N, L, C, G)
    # the decoder shapes: one statistics workgroup per CU of an MI355X
    for N, L, C, G in SHAPES[:5]:
        assert gn.plan_rows(N, L, C, G)["K1"] == 256


def test_plan_declines_like_the_entry_points():
    assert gn.plan_rows(1, 16, 96, 32) is None        # C not a power of two
    assert gn.plan_rows(1, 16, 4096, 32) is None      # C > 2048
    with pytest.raises(ValueError):
        gn.plan_rows(1, 16, 64, 3)                    # C % G != 0
    assert gn.plan_rows(0, 16, 64, 32)["K1"] == 0     # empty: nothing launched


def test_slot_maps_are_permutations_of_a_tile():
    """Lane tid's slot j holds element o(tid, j) of each 2048-element tile:
    8*tid + j for 16-bit types, 4*tid + j and 1024 + 4*tid + (j - 4) for
    fp32.  Each map must cover the tile exactly once, and each 16-byte access
    (4 fp32 / 8 16-bit slots) must be contiguous and 16-byte aligned."""
    def o16(tid, j):
        return 8 * tid + j

    def o32(tid, j):
        return (0 if j < 4 else 1024 - 4) + 4 * tid + j

    for o, per_access in ((o16, 8), (o32, 4)):
        offs = [o(t, j) for t in range(THREADS) for j in range(8)]
        assert sorted(offs) == list(range(THREADS * 8))
        for t in range(THREADS):
            for a in range(0, 8, per_access):
                run = [o(t, j) for j in range(a, a + per_access)]
                assert run == list(range(run[0], run[0] + per_access))
                assert run[0] % per_access == 0
        # one wave instruction (64 lanes, same access index) covers 1 KiB contiguously
        for a in range(0, 8, per_access):
            for w in range(THREADS // 64):
                starts = sorted(o(t, a) for t in range(64 * w, 64 * w + 64))
                assert starts == list(range(starts[0], starts[0] + 64 * per_access, per_access))

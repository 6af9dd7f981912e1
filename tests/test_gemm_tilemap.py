"""The grouped GEMM's tile order, modelled on the host: tile number -> (expert,
row tile, column tile) as map_tile in csrc/expert_gemm.hip states it.

Model: expert e has mt_e = ceil(n_e / 256) row tiles and NT column tiles;
its tiles are numbered after those of experts 0 .. e-1.  Within an expert, row
blocks of RBLOCK = 4 row tiles (the last may be short) are walked in groups of
NGROUP = 8 column tiles, row tile by row tile within a group.  Workgroups go to
the 8 XCDs in turn by tile number.  Checked: every (expert, row tile, column
tile) is numbered exactly once, and, where NT is a multiple of 8 (every
Mixtral projection: 112 and 16 column tiles), the row tiles of one column
inside a group run on one XCD, so that they share that weight tile in one L2."""
import itertools

import pytest

BM, NGROUP, RBLOCK, XCDS = 256, 8, 4, 8


def map_tile(counts, NT, L):
    cum = 0
    for e, n_e in enumerate(counts):
        mt = (n_e + BM - 1) // BM
        cnt = mt * NT
        if L < cum + cnt:
            i = L - cum
            rb = i // (RBLOCK * NT)
            rbr = min(RBLOCK, mt - rb * RBLOCK)
            ib = i - rb * RBLOCK * NT
            g = ib // (rbr * NGROUP)
            gi = ib - g * rbr * NGROUP
            gw = min(NGROUP, NT - g * NGROUP)
            m = rb * RBLOCK + gi // gw
            nn = gi - (gi // gw) * gw
            return e, m, g * NGROUP + nn, (rb, g)
        cum += cnt
    return None


def tiles(counts, NT):
    return sum((c + BM - 1) // BM for c in counts) * NT


@pytest.mark.parametrize("NT", [1, 3, 8, 16, 24, 112, 113])
def test_every_tile_numbered_once(NT):
    for mts in itertools.product(range(0, 10), repeat=2):
        counts = [m * BM - (7 if m else 0) for m in mts] + [1]
        got = [map_tile(counts, NT, L)[:3] for L in range(tiles(counts, NT))]
        want = {(e, m, n) for e, c in enumerate(counts) for m in range((c + BM - 1) // BM) for n in range(NT)}
        assert len(got) == len(set(got)) and set(got) == want, (NT, mts)


@pytest.mark.parametrize("counts", [
    [1023, 1045, 1008, 1024, 1003, 1055, 1004, 1030],      # the T = 4096 layer
    [11503, 6995, 4592, 3092, 2372, 1753, 1400, 1061],     # the Zipf-skewed T = 16384 layer
    [0, 8192, 0, 0, 0, 0, 0, 0],
])
@pytest.mark.parametrize("NT", [112, 16])
def test_group_columns_stay_on_one_xcd(counts, NT):
    seen = {}
    for L in range(tiles(counts, NT)):
        e, m, n, grp = map_tile(counts, NT, L)
        seen.setdefault((e, grp, n), set()).add(L % XCDS)
    assert all(len(x) == 1 for x in seen.values())

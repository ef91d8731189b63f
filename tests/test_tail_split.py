"""Coverage of the grouped GEMM's work split (CPU only).

The big-tile GEMM launches of one projection split their units (expert tile,
block of 32 weight groups) between a launch of 64 x 512 tiles and, for each
XCD's last round when it fits the XCD's compute units as halves, a launch of
64 x 256 tiles that runs each such unit as two half-width units (where the
weight groups do not split into blocks of 32, one launch of 64 x 256 tiles). This test restates the kernel's unit
decode (expert_gemm_kernel's prologue and tail_split in gemm.hpp) and the
host's launch choices (forward_layer in moe_ffn.hip) in Python, enumerates
every workgroup of the launches, and checks that every (tile, weight group) of
the output is computed exactly once and that no workgroup reads a tile past
the tile list: over a sweep of tile counts, column blocks and CUs per XCD, and
on the tile counts that the 30b prefill and 235b routings produce.
"""
import numpy as np
import pytest

import synth

GEMM_M = 64            # rows of a big tile
GEMM_MIN_ROWS = 17     # buckets of at least this many pairs take big tiles
GROUPS_FULL = 32       # weight groups of a 64 x 512 unit
GROUPS_HALF = 16       # weight groups of a 64 x 256 unit


def tail_split(ntl, ncb, x, C):
    per_xcd = (ntl + 7) >> 3
    n_x = max(0, min(per_xcd, ntl - x * per_xcd)) * ncb
    r = n_x % C if C > 0 else 0
    r_x = r if (r > 0 and 2 * r <= C) else 0
    return per_xcd, n_x - r_x, r_x


def max_gemm_tiles(S, E):
    big_buckets = min(S // GEMM_MIN_ROWS, E)
    return S // GEMM_M + big_buckets


def units_of_launch(ntl, ngroups, groups, grid, mode, C):
    """(tile, first group, groups) of every workgroup of one launch that does work."""
    out = []
    for bid in range(grid):
        x, sid = bid & 7, bid >> 3
        if mode == 2:
            ncb8 = ngroups // (2 * groups)
            per_xcd, full_x, r_x = tail_split(ntl, ncb8, x, C)
            if sid >= 2 * r_x:
                continue
            u = full_x + (sid >> 1)
            tile = x * per_xcd + u // ncb8
            rg0 = (u % ncb8) * 2 * groups + (sid & 1) * groups
        else:
            ncb = ngroups // groups
            per_xcd, full_x, _ = tail_split(ntl, ncb, x, C if mode == 1 else 0)
            if sid >= full_x:
                continue
            tile = x * per_xcd + sid // ncb
            rg0 = (sid % ncb) * groups
        out.append((tile, rg0, groups))
    return out


def big_launches(ntl, S, E, ngroups, cus_per_xcd):
    """The host's big-tile launches of one projection: [(groups per unit, grid, mode, C)]."""
    C = cus_per_xcd if S >= E * GEMM_MIN_ROWS else 0
    mg8 = (max_gemm_tiles(S, E) + 7) // 8
    if ngroups % 32 == 0:  # 64 x 512 tiles, the last round's split units as halves
        ls = [(GROUPS_FULL, 8 * (ngroups // GROUPS_FULL) * mg8, 1, C)]
        if C > 0:
            ls.append((GROUPS_HALF, 8 * C, 2, C))
        return ls
    return [(GROUPS_HALF, 8 * (ngroups // GROUPS_HALF) * mg8, 0, 0)]


def check_cover(ntl, S, E, ngroups, cus_per_xcd):
    seen = np.zeros((max(ntl, 1), ngroups), np.int32)
    for groups, grid, mode, C in big_launches(ntl, S, E, ngroups, cus_per_xcd):
        for tile, rg0, g in units_of_launch(ntl, ngroups, groups, grid, mode, C):
            assert 0 <= tile < ntl, (tile, ntl, mode)
            assert 0 <= rg0 and rg0 + g <= ngroups
            seen[tile, rg0:rg0 + g] += 1
    assert np.all(seen[:ntl] == 1), np.argwhere(seen[:ntl] != 1)[:5]


def test_tail_split_counts():
    # 100 tiles x 3 column blocks over 8 XCDs of 32 CUs: 13 tiles (39 units)
    # per XCD, 7 left over in the last round -> split into 14 halves
    assert tail_split(100, 3, 0, 32) == (13, 32, 7)
    # the last XCD has 100 - 7 * 13 = 9 tiles = 27 units: 27 > 16, not split
    assert tail_split(100, 3, 7, 32) == (13, 27, 0)
    # no CUs given: nothing split
    assert tail_split(100, 3, 0, 0) == (13, 39, 0)
    # an XCD past the end of the tile list has no units
    assert tail_split(3, 3, 5, 32) == (1, 0, 0)


@pytest.mark.parametrize("cus", [32, 30, 16, 8, 4, 1])
@pytest.mark.parametrize("ngroups", [32, 64, 96, 128, 192, 256, 48, 80])
def test_every_tile_and_group_once(cus, ngroups):
    E = 128
    for ntl in list(range(1, 70)) + [100, 127, 255, 256, 257, 300, 511]:
        # the smallest pair count that yields ntl tiles, and a large one
        for S in (ntl * GEMM_M, E * GEMM_MIN_ROWS + ntl * GEMM_M):
            if max_gemm_tiles(S, E) >= ntl:
                check_cover(ntl, S, E, ngroups, cus)


@pytest.mark.parametrize("name", ["30b-prefill", "235b-shape", "30b-batch"])
def test_workload_routings(name):
    """Tile counts of the workloads' own routing (the oracle's top-k on the seeded inputs), gate/up and down."""
    import oracle

    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl, seed=0)
    _, idx, _ = oracle.router(inp.x, inp.router, inp.bias, wl.top_k)
    cnt = np.bincount(idx.ravel(), minlength=wl.experts)
    ntl = int(sum((c + GEMM_M - 1) // GEMM_M for c in cnt if c >= GEMM_MIN_ROWS))
    S = wl.tokens * wl.top_k
    assert ntl <= max_gemm_tiles(S, wl.experts)
    for ngroups in (wl.inter // 8, wl.hidden // 16):
        for cus in (32, 30):
            check_cover(ntl, S, wl.experts, ngroups, cus)
    if name == "30b-prefill":
        # the case that mixes both modes: with 274 tiles, XCDs 0-6 (35 tiles x 3 column blocks = 105 units on 32
        # CUs) split a last round of 9 units into halves, XCD 7 (29 tiles, 87 units) leaves its 23 whole
        split = [tail_split(ntl, wl.inter // 8 // GROUPS_FULL, x, 32)[2] for x in range(8)]
        assert ntl == 274 and split == [9] * 7 + [0], (ntl, split)

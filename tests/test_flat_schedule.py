"""The flat decode schedule's team ranges (CPU only).

The flat kernel deals the tile stream in periods of Q = 2 TW teams (the TW
teams of two consecutive workgroups) of P = Q per tiles; team q of a period
takes [off(q), off(q + 1)), the offsets in proportion to integer weights: the
first workgroup of the pair kXcdPct (kXcdPctMfma or kXcdPctValu), the second
the rest, and inside a workgroup of two teams the first kSplitPct, else equal
shares.  The merge pass reads one record per team from the first to the last
team holding a split (sequence, head group) pair, so every team of a period
must hold at least one tile: a team with none would leave its record
unwritten.  The weights are constants of the kernel source; this reads them
there and checks, for every period the launcher can form, that the offsets
run from 0 to P and rise strictly, and that the owner the merge computes for
a tile is the team whose range holds it.
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECODE = os.path.join(ROOT, "paged_kv_cache_227_amd", "csrc", "decode.hip")


def _const(name):
    src = open(DECODE, encoding="utf-8").read()
    m = re.search(r"constexpr int %s = (\d+);" % name, src)
    assert m, "%s not found in decode.hip" % name
    return int(m.group(1))


def offsets(TW, P, split, xcd):
    """off(0) .. off(Q): integer weights, rounded down like the kernel's
    64-bit P * cum / total."""
    def in_wg(n):  # weight of the first n teams of a workgroup
        if TW == 2:
            return 0 if n <= 0 else (split if n == 1 else 100)
        return 50 * n
    tot = 100 * in_wg(TW)
    return [P * (xcd * in_wg(min(q, TW)) + (100 - xcd) * in_wg(max(q - TW, 0))) // tot for q in range(2 * TW + 1)]


def owner(t, P, off):
    """The merge's piece(t): the last team of t's period whose offset is at or below t mod P."""
    r = t % P
    return (t // P) * (len(off) - 1) + sum(1 for i in range(1, len(off) - 1) if off[i] <= r)


# Teams per workgroup the launchers form: the matrix-core tune (8 waves, teams
# of up to 4, fewer when the head groups do not divide) and the vector tunes
# (4 waves, teams of one); the in-workgroup split applies to two teams only.
TEAMS = [(2, "kXcdPctMfma"), (4, "kXcdPctMfma"), (8, "kXcdPctMfma"), (4, "kXcdPctValu")]


@pytest.mark.parametrize("TW,xcd_name", TEAMS)
def test_every_team_holds_tiles(TW, xcd_name):
    split = _const("kSplitPct") if TW == 2 else 50
    xcd = _const(xcd_name)
    assert 0 < split < 100 and 0 < xcd < 100
    Q = 2 * TW
    for per in range(1, 4097):
        P = Q * per
        off = offsets(TW, P, split, xcd)
        assert off[0] == 0 and off[-1] == P
        assert all(b > a for a, b in zip(off, off[1:])), "a team of a %d-tile period holds no tile: %s" % (P, off)


@pytest.mark.parametrize("TW,xcd_name", TEAMS)
def test_merge_finds_each_tiles_team(TW, xcd_name):
    split = _const("kSplitPct") if TW == 2 else 50
    xcd = _const(xcd_name)
    Q = 2 * TW
    for per in (1, 2, 3, 7, 64, 301):
        P = Q * per
        off = offsets(TW, P, split, xcd)
        for t in range(3 * P):
            team = owner(t, P, off)
            j, q = divmod(team, Q)
            assert j * P + off[q] <= t < j * P + off[q + 1]


def test_offsets_pin():
    """A worked period: 4 teams (two workgroups of two), 100 tiles, the first
    workgroup 52 %, inside each the first team 62 %: shares of 32.24, 19.76,
    29.76 and 18.24 tiles, each offset rounded down."""
    assert offsets(2, 100, 62, 52) == [0, 32, 52, 81, 100]

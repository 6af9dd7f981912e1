"""The grouped GEMM's LDS ring schedule, modelled on the host: no copy into a
ring slot may be issued before every operand read of the rows it overwrites
(in the slot's previous slice) is complete.

Model (as csrc/expert_gemm.hip states it): a ring of NS = 5 slots per operand,
each slot 256 rows in 16-row groups; a copy instruction of wave w covers rows
64 w + 16 j .. + 15 for its row group j.  Wave group g runs the memory phase of
K slice s in interval 2s + g and its compute phase in the interval after; each
memory phase reads slot s % NS of both operands' rings (group g's A reads:
rows 128 g + 16 mi, blocks mi = 0, 1, 4, 5 first), and group 0 copies operand
A, group 1 operand B: at an odd s row groups 0, 1 of slices s+3 and s+4, at an
even s row groups 2, 3 of slices s+2 and s+3.  A read is complete at the end of
its memory phase if that phase waits for it (lgkmcnt), else at the end of its
compute phase, whose MFMAs wait for every operand they use.  The kernel waits
in group 1's even steps, for the four A reads it issues first."""
import pytest

NS = 5
EARLY = (0, 1, 4, 5)  # A blocks read first
LATE = (2, 3, 6, 7)


def row_group(row):
    """Row group j (0..3) of the copy instruction that writes this slot row."""
    return (row % 64) // 16


def hazards(KT, waits_early):
    """waits_early(g, s): group g's memory phase of slice s waits for its first
    four A reads (blocks 0, 1, 4, 5)."""
    reads, copies = [], []
    for g in (0, 1):
        for s in range(KT):
            mem = 2 * s + g
            for blocks, early in ((EARLY, True), (LATE, False)):
                done = mem if (early and waits_early(g, s)) else mem + 1
                rgs = {row_group(128 * g + 16 * mi) for mi in blocks}
                reads.append(("A", s, frozenset(rgs), done))
            reads.append(("B", s, frozenset(range(4)), mem + 1))
            ring = "A" if g == 0 else "B"
            targets, rgs = ((s + 3, s + 4), {0, 1}) if s % 2 else ((s + 2, s + 3), {2, 3})
            for t in targets:
                copies.append((ring, t, frozenset(rgs), mem))
    out = []
    for ring, t, crg, issue in copies:
        for r_ring, q, rrg, done in reads:
            if r_ring == ring and q == t - NS and (crg & rrg) and issue < done + 1:
                out.append((ring, t, issue, q, done))
    return out


def kernel_waits(g, s):
    return g == 1 and s % 2 == 0


@pytest.mark.parametrize("KT", [2, 4, 6, 10, 26, 128, 448])
def test_ring_schedule_has_no_copy_over_pending_reads(KT):
    assert hazards(KT, kernel_waits) == []


def test_the_kept_waits_are_needed():
    # Without any read wait, group 0's odd-step copy reaches rows that group 1
    # has just read at an even step.
    found = hazards(26, lambda g, s: False)
    assert found and all(ring == "A" and q % 2 == 0 and issue == done for ring, _, issue, q, done in found)
    # Dropping the wait at any single even step of group 1 opens exactly that slice.
    for s in range(0, 24, 2):
        found = hazards(26, lambda g, t, s=s: kernel_waits(g, t) and not (g == 1 and t == s))
        assert [(q, ring) for ring, _, _, q, _ in found] == [(s, "A")]


def test_the_early_blocks_hold_the_rows_copied_one_interval_later():
    # The rows that an odd-step copy writes (row groups 0, 1) are exactly the
    # rows of the blocks issued first, in both wave rows; the others are not.
    for g in (0, 1):
        assert {row_group(128 * g + 16 * mi) for mi in EARLY} == {0, 1}
        assert {row_group(128 * g + 16 * mi) for mi in LATE} == {2, 3}

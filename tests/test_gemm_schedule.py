"""The grouped GEMM's LDS ring schedule, modelled on the host: no copy into a
ring slot may be issued before every operand read of the slot's previous
slice is complete.

Model (as csrc/expert_gemm.hip states it): a ring of NS = 5 slots per operand;
wave group g runs the memory phase of K slice s in interval 2s + g and its
compute phase in the interval after; each memory phase reads slot s % NS of
both operands' rings, and group 0 copies operand A, group 1 operand B: at an
odd s row groups 0, 1 of slices s+3 and s+4, at an even s row groups 2, 3 of
slices s+2 and s+3.  A group's reads are complete at the end of its memory
phase if it waits for them there (lgkmcnt), else at the end of its compute
phase, whose MFMAs wait for every operand they use.  The kernel waits in
group 1's even steps only."""
import pytest

NS = 5


def hazards(KT, waits):
    reads, copies = [], []
    for g in (0, 1):
        for s in range(KT):
            mem = 2 * s + g
            done = mem if waits(g, s) else mem + 1
            for ring in "AB":
                reads.append((ring, s, done))
            targets = (s + 3, s + 4) if s % 2 else (s + 2, s + 3)
            for t in targets:
                copies.append(("A" if g == 0 else "B", t, mem))
    out = []
    for ring, t, issue in copies:
        for r_ring, q, done in reads:
            if r_ring == ring and q == t - NS and issue < done + 1:
                out.append((ring, t, issue, q, done))
    return out


def kernel_waits(g, s):
    return g == 1 and s % 2 == 0


@pytest.mark.parametrize("KT", [2, 4, 6, 10, 26, 128, 448])
def test_ring_schedule_has_no_copy_over_pending_reads(KT):
    assert hazards(KT, kernel_waits) == []


def test_each_wait_the_kernel_keeps_is_needed():
    # Without any read wait, group 0's odd-step copy reaches the slot group 1
    # has just read at an even step.
    found = hazards(26, lambda g, s: False)
    assert found and all(ring == "A" and q % 2 == 0 and issue == done for ring, _, issue, q, done in found)
    # Dropping the wait at any single even step of group 1 opens exactly that slot.
    for s in range(0, 24, 2):
        found = hazards(26, lambda g, t, s=s: kernel_waits(g, t) and not (g == 1 and t == s))
        assert [(q, ring) for ring, _, _, q, _ in found] == [(s, "A")]

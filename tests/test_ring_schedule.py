"""CPU check of the schedule of the index ring in the weight-gradient GEMMs
(csrc/gemm.hip, kDW with a gathered operand).

The kernel keeps the token-row offsets of an expert's rows in a ring of 3
slots of one chunk each (RING_STAGES stages of rows per chunk).  Its rules,
restated here:
  - stage kt covers row block kt (one pass), or kt // 2 when the operand is
    split (hi and lo stages of each block alternate); chunk sequence number of
    stage kt: its block // CS; chunk q lives in slot q % 3;
  - with L2 prefetch distance P (1 or 2), RA = 2 + P;
  - before the first stage: load the chunks of stages 0 .. RA - 1, wait,
    barrier;
  - at stage kt (when a next stage exists), after the stage's wait + barrier:
    load the chunk that stage kt + RA starts, if it starts one; then read the
    offsets for stage kt + 1 (its loads) and stage min(kt + 1 + P, nk - 1)
    (the L2 prefetch touch);
  - a load issued at stage s has completed (and is visible to every wave) at
    stage s + 1, after that stage's wait and barrier.
Every read must find its chunk in its slot, written by a load that completed
before the read, and no load may target a slot that a read of the same stage
uses.
"""
import pytest


def simulate(nk_pass, split, cs, prefetch=1, slots=3):
    nk = 2 * nk_pass if split else nk_pass

    def q(kt):
        return (kt // 2 if split else kt) // cs

    slot = {}

    def load(c, stage):
        slot[c % slots] = (c, stage)

    def read(kt, stage):
        c = q(kt)
        got = slot.get(c % slots)
        assert got is not None and got[0] == c, (nk_pass, split, cs, stage, kt, c, got)
        assert got[1] < stage, ("read of a load still in flight", nk_pass, split, cs, stage, kt)

    if nk == 0:
        return 0
    ra = 2 + prefetch
    for s in range(min(ra, nk)):
        if s == 0 or q(s) != q(s - 1):
            load(q(s), -2)
    read(0, -1)
    read(min(prefetch, nk - 1), -1)
    reads = 2
    for kt in range(nk):
        if kt + 1 < nk:
            if kt + ra < nk and q(kt + ra) != q(kt + ra - 1):
                load(q(kt + ra), kt)
            read(kt + 1, kt)
            read(min(kt + 1 + prefetch, nk - 1), kt)
            reads += 2
    return reads


@pytest.mark.parametrize("cs", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("prefetch", [1, 2])
def test_ring_schedule_every_stage_count(cs, prefetch):
    if prefetch == 2 and cs < 2:
        pytest.skip("distance 2 needs chunks of at least 2 stages (the kernel's are 8 or more)")
    for nk_pass in range(0, 160):
        for split in (False, True):
            simulate(nk_pass, split, cs, prefetch=prefetch)


def test_ring_schedule_distance_two_needs_two_stage_chunks():
    """With one-stage chunks the distance-2 schedule overwrites a chunk still in
    use, which is why the kernel asserts its chunks span the distance."""
    with pytest.raises(AssertionError):
        for nk_pass in range(0, 64):
            simulate(nk_pass, False, 1, prefetch=2)


def test_ring_schedule_needs_three_slots():
    """With two slots the same rules fail (a chunk is overwritten while a stage
    in flight still reads it), so the third slot is what makes them safe."""
    with pytest.raises(AssertionError):
        for nk_pass in range(0, 64):
            for split in (False, True):
                simulate(nk_pass, split, 1, slots=2)

"""Host-side model of the grouped GEMM's load/wait schedule (no GPU).

The persistent GEMM keeps two LDS stage rings (gathered A rows NA deep,
weight rows NB deep) running continuously across a workgroup's tiles.  Step j
of tile i issues A(j+NA-1) then B(j+NB-1) (slabs of the next tile once the
index runs past K), each as a fixed number of loads per wave; every tile ends
with a fixed number of epilogue stores.  Vector-memory operations retire in
issue order, and before computing a slab a wave waits until at most WAIT
operations (WAIT + STORES at a tile's first step after an epilogue) are
pending.  This model replays that schedule for many ring depths and load
counts and checks that every wait really covers the slab about to be read,
that each slab sits in the stage it is read from, and that no stage is
refilled while it is being read.  The staged epilogue writes a tile's output
into the A and B stages its last step read: the model checks that those two
stages hold nothing still needed and that no load is landing in them then.
The WAIT formula below is the one the kernel computes at compile time.
"""
import pytest


def wait_count(NA, NB, A_INST, B_INST):
    LOADS = A_INST + B_INST
    return B_INST + (NA - 2) * LOADS if NA < NB else (NB - 2) * LOADS


def replay(KT, NA, NB, A_INST, B_INST, STORES, ntiles, staging_offset=1):
    """staging_offset: the epilogue stages into the stages `staging_offset`
    steps behind the read pointers (1: the ones the last step read)."""
    WAIT = wait_count(NA, NB, A_INST, B_INST)
    pending = []                 # (kind, slab, stage), oldest first
    stage_a, stage_b = {}, {}

    def issue(kind, stage, slab):
        (stage_a if kind == "A" else stage_b)[stage] = slab
        pending.extend([(kind, slab, stage)] * (A_INST if kind == "A" else B_INST))

    def wait(n):
        del pending[:max(0, len(pending) - n)]

    lead = max(NA, NB)
    for j in range(-(lead - 1), 0):          # prologue of the first tile
        if j + NA - 1 >= 0:
            issue("A", j + NA - 1, (0, j + NA - 1))
        if j + NB - 1 >= 0:
            issue("B", j + NB - 1, (0, j + NB - 1))
    a_read = b_read = 0
    for tile in range(ntiles):
        nxt = tile + 1 if tile + 1 < ntiles else None
        for kt in range(KT):
            wait(WAIT + STORES if (kt == 0 and tile > 0) else WAIT)
            assert stage_a.get(a_read) == (tile, kt) and stage_b.get(b_read) == (tile, kt)
            assert all(p[:2] not in (("A", (tile, kt)), ("B", (tile, kt))) for p in pending)
            # the barrier retires slab kt-1: its stages are refilled now
            a_fill, b_fill = (a_read - 1) % NA, (b_read - 1) % NB
            assert a_fill != a_read and b_fill != b_read
            ta, tb = kt + NA - 1, kt + NB - 1
            issue("A", a_fill, (tile, ta) if ta < KT else (nxt, ta - KT))
            issue("B", b_fill, (tile, tb) if tb < KT else (nxt, tb - KT))
            a_read, b_read = (a_read + 1) % NA, (b_read + 1) % NB
        # staged epilogue (after a barrier): the stages the last step read
        sa, sb = (a_read - staging_offset) % NA, (b_read - staging_offset) % NB
        assert stage_a.get(sa) == (tile, KT - 1) and stage_b.get(sb) == (tile, KT - 1), \
            "the staging stages still hold a slab to be read"
        assert not any((p[0], p[2]) in (("A", sa), ("B", sb)) for p in pending), \
            "a load is still landing in a staging stage"
        pending.extend([("S", tile, None)] * STORES)


@pytest.mark.parametrize("NA", [2, 3, 4])
@pytest.mark.parametrize("NB", [2, 3, 4, 5, 6])
def test_waits_cover_every_slab(NA, NB):
    for KT in range(max(NA, NB - 1), 34):
        for a_inst, b_inst, stores in [(4, 4, 8), (4, 4, 16), (1, 4, 2), (2, 8, 4), (8, 8, 32)]:
            if wait_count(NA, NB, a_inst, b_inst) + stores >= 64:
                continue                     # beyond the 6-bit vmcnt field; the kernel asserts it
            for ntiles in (1, 2, 3, 5):
                replay(KT, NA, NB, a_inst, b_inst, stores, ntiles)


def test_a_looser_wait_is_caught():
    """The model is strict enough to notice a wait one operation too loose."""
    global wait_count
    orig = wait_count
    try:
        wait_count = lambda NA, NB, a, b: orig(NA, NB, a, b) + 1   # noqa: E731
        with pytest.raises(AssertionError):
            replay(8, 2, 3, 4, 4, 8, 2)
    finally:
        wait_count = orig


def test_staging_in_the_next_stages_is_caught():
    """Staging the output in the stages the read pointers already moved to
    (which hold the next tile's first slab) fails the model."""
    replay(8, 2, 3, 4, 4, 8, 3)
    with pytest.raises(AssertionError):
        replay(8, 2, 3, 4, 4, 8, 3, staging_offset=0)

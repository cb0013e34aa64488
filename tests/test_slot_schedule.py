"""Host-side model of the slot GEMM's producer/consumer schedule (no GPU).

One persistent workgroup walks S = tiles x KT K steps.  The A ring has two
stages and the B (weight) ring three.  Producer waves issue B(0), A(0), B(1)
before the first barrier, then at step g refill A(g+1) into the A stage the
consumers read at step g-1 and B(g+2) into the B stage they read at step g-1,
wait until at most B_INST of their own loads are pending and meet the
consumers at the step's barrier.  Consumers read slab g from A stage g % 2 and
B stage g % 3 between barrier g and barrier g+1 and never wait on the memory
counter.  Loads retire in issue order.  At the last step of a tile both kinds
of wave pass one barrier more: between the two, the consumers stage the
tile's output in the A and B stages that step read.  The replay follows the
kernel's own stage-offset arithmetic and checks, for several load counts and
tile walks, that after every barrier the slab the consumers read next is
complete and sits in the stages they read, that no stage is refilled while it
is read, that no load is still landing in (or issued into) a stage while the
output is staged there, and that both kinds of wave pass the same number of
barriers; a looser wait is shown to expose a slab, and a refill issued before
the extra barrier to land on the staged output.
"""
import pytest

NA, NB = 2, 3


def replay(A_INST, B_INST, KT, ntiles, wait=None, early_refill=False):
    """Returns None if the schedule is sound, else a description of the
    first violation.  early_refill: the producers skip the extra barrier at
    a tile's end (a broken schedule)."""
    S = ntiles * KT
    WAIT = B_INST if wait is None else wait
    A_STAGE, B_STAGE = 1, 1                 # offsets in units of one stage
    pending = []                            # (operand, slab, stage), oldest first
    a_stage, b_stage = {}, {}               # stage offset -> slab it holds (or is loading)

    def issue(op, slab, off):
        (a_stage if op == "A" else b_stage)[off] = slab
        pending.extend([(op, slab, off)] * (A_INST if op == "A" else B_INST))

    def wait_until(n):
        del pending[:max(0, len(pending) - n)]

    def landed(op, slab):
        return all((o, s) != (op, slab) for o, s, _ in pending)

    # producer prologue: B(0) -> B stage 0, A(0) -> A stage 0, B(1) -> B stage 1
    issue("B", 0, 0)
    issue("A", 0, 0)
    issue("B", 1, B_STAGE)
    wait_until(WAIT)
    barriers = {"producer": 1, "consumer": 1}
    a_fill, b_fill = A_STAGE, 2 * B_STAGE
    a_rd, b_rd = 0, 0
    for g in range(S):
        # consumers read slab g between barrier g and barrier g+1
        if a_stage.get(a_rd) != g or b_stage.get(b_rd) != g:
            return f"step {g}: stages hold A{a_stage.get(a_rd)} B{b_stage.get(b_rd)}"
        if not (landed("A", g) and landed("B", g)):
            return f"step {g}: slab read before it landed"
        # producers refill the stages computed at step g-1
        if a_fill == a_rd or b_fill == b_rd:
            return f"step {g}: a stage is refilled while it is read"
        issue("A", g + 1, a_fill)
        issue("B", g + 2, b_fill)
        a_fill = A_STAGE if a_fill == 0 else 0
        b_fill = 0 if b_fill + B_STAGE == NB * B_STAGE else b_fill + B_STAGE
        wait_until(WAIT)
        barriers["producer"] += 1
        tile_end = (g + 1) % KT == 0
        if tile_end:
            # after the extra barrier the consumers stage the output in the
            # stages step g read: nothing may still land there, and the
            # producers issue nothing until the next barrier
            # (the stages the producers fill next, at step g+1)
            if early_refill and g + 1 < S and (a_fill == a_rd or b_fill == b_rd):
                return f"step {g}: a refill lands on the staged output"
            if any(st == a_rd for o, _, st in pending if o == "A") or \
               any(st == b_rd for o, _, st in pending if o == "B"):
                return f"step {g}: a load is still landing on the staged output"
            if not early_refill:
                barriers["producer"] += 1
        # consumers advance their read offsets, then meet at the barrier
        # (two at a tile's end)
        a_rd = A_STAGE if a_rd == 0 else 0
        b_rd = 0 if b_rd + B_STAGE == NB * B_STAGE else b_rd + B_STAGE
        barriers["consumer"] += 2 if tile_end else 1
    if barriers["producer"] != barriers["consumer"] or barriers["producer"] != S + 1 + ntiles:
        return f"barrier counts differ: {barriers}"
    return None


@pytest.mark.parametrize("A_INST,B_INST", [(8, 8), (4, 8), (8, 4), (1, 1), (2, 5)])
@pytest.mark.parametrize("KT", [1, 2, 3, 4, 32])
@pytest.mark.parametrize("ntiles", [1, 2, 5])
def test_producer_waits_cover_every_slab(A_INST, B_INST, KT, ntiles):
    assert replay(A_INST, B_INST, KT, ntiles) is None


def test_the_kernels_load_counts():
    """256x256 tiles of 64-deep slabs, four producer waves, 1 KB per load:
    A (256 rows x 128 B) and B (256 rows x 128 B, or 64 K rows x 512 B) are
    32 KB stages, eight loads per producer wave each."""
    A_INST = 256 * 64 * 2 // 1024 // 4
    B_INST = 64 * 256 * 2 // 1024 // 4
    assert (A_INST, B_INST) == (8, 8)
    assert replay(A_INST, B_INST, 12, 4) is None


def test_looser_wait_exposes_a_slab():
    """Allowing A's loads to stay pending as well lets the consumers read an
    A slab that has not landed, so the check has teeth."""
    A_INST, B_INST = 8, 8
    assert replay(A_INST, B_INST, 4, 3, wait=B_INST) is None
    assert replay(A_INST, B_INST, 4, 3, wait=B_INST + A_INST) is not None


def test_refill_before_the_extra_barrier_hits_the_staged_output():
    """Without the producers' extra barrier at a tile's end, their next
    refill goes into a stage the consumers are staging the output in."""
    assert replay(8, 8, 4, 3) is None
    assert replay(8, 8, 4, 3, early_refill=True) is not None

"""Host-side model of the weight-gradient kernel's producer/consumer schedule
(no GPU).

One persistent workgroup walks S = tiles x KT K steps.  Producer waves issue
the loads of slab g+D-1 (A then B, INST loads each) into the stage the
consumers computed at step g-1, then wait until at most WAIT of their own
loads are pending and meet the consumers at the step's barrier; consumers
read slab g from stage g % D between barrier g and barrier g+1 and never wait
on the memory counter (their stores do not enter the producers' counts).
Loads retire in issue order.  The replay checks, for ring depths 2..5, that
after every barrier the slab the consumers read next is complete and sits in
the stage they read, that no stage is refilled while it is being read, and
that both kinds of wave pass the same number of barriers.  WAIT is the
formula the kernel computes at compile time.
"""
import pytest


def wait_count(D, INST):
    # a producer's loads issued after slab g+1's when it waits for that slab
    return (D - 2) * 2 * INST


def replay(D, INST, KT, ntiles):
    S = ntiles * KT
    WAIT = wait_count(D, INST)
    pending = []                      # the producer's loads, oldest first
    stage = {}                        # stage -> slab held (A and B move together)
    barriers = {"producer": 0, "consumer": 0}

    def issue(slab, st):
        stage[st] = slab
        pending.extend([("A", slab)] * INST + [("B", slab)] * INST)

    def wait(n):
        del pending[:max(0, len(pending) - n)]

    def landed(slab):
        return all(s != slab for _, s in pending)

    # producer prologue: slabs 0 .. D-2 into stages 0 .. D-2, wait for slab 0
    for j in range(D - 1):
        issue(j, j)
    wait(WAIT)
    barriers["producer"] += 1
    barriers["consumer"] += 1                       # barrier 0
    fill = D - 1
    for g in range(S):
        # between barrier g and g+1: consumers read slab g from stage g % D
        read = g % D
        assert stage.get(read) == g, (g, stage)
        assert landed(g), f"slab {g} read before it landed"
        # producers refill the stage the consumers read at step g-1
        assert fill != read
        issue(g + D - 1, fill)
        fill = (fill + 1) % D
        wait(WAIT)
        # at barrier g+1 the next slab must be complete
        if g + 1 < S:
            assert landed(g + 1), f"slab {g + 1} incomplete at barrier {g + 1}"
        barriers["producer"] += 1
        barriers["consumer"] += 1
    assert barriers["producer"] == barriers["consumer"] == S + 1


@pytest.mark.parametrize("D", [2, 3, 4, 5])
@pytest.mark.parametrize("INST", [1, 2, 4, 8])
@pytest.mark.parametrize("KT", [1, 2, 3, 4, 7])
def test_producer_waits_cover_every_slab(D, INST, KT):
    replay(D, INST, KT, ntiles=5)


def test_shallower_wait_would_expose_a_slab():
    """The formula is tight: allowing one more pending load than it leaves
    exposes a slab that has not landed (so the check has teeth)."""
    D, INST, KT = 3, 4, 4
    good = wait_count(D, INST)

    def replay_with(w):
        pending, stage = [], {}

        def issue(slab, st):
            stage[st] = slab
            pending.extend([slab] * (2 * INST))

        def wait(n):
            del pending[:max(0, len(pending) - n)]

        for j in range(D - 1):
            issue(j, j)
        wait(w)
        fill = D - 1
        for g in range(KT * 3):
            if g in pending:
                return False
            issue(g + D - 1, fill)
            fill = (fill + 1) % D
            wait(w)
        return True

    assert replay_with(good)
    assert not replay_with(good + 1)

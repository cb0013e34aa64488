"""Host logic of the variable-N serving ladder ([BK] "What this adds"): the
bucket sizes, the choice of bucket for an item and the eager fallback, and
the free-memory bound on capture.  No device work."""

import pytest

from mixture_experts_expert_amd.serving import DEFAULT_FACTORS, BucketLadder


def test_ladder_sizes_cluster_above_half_and_one():
    L = BucketLadder(4096, 8192)
    assert L.sizes == sorted(set(L.sizes)) and L.sizes[-1] == 8192
    assert all(s % 16 == 0 for s in L.sizes)
    # every factor's size is present, capped at the ceiling
    for f in DEFAULT_FACTORS:
        want = min(8192, -(-int(-(-f * 4096 // 1)) // 16) * 16)
        assert want in L.sizes, f
    near_half = [s for s in L.sizes if 2048 <= s <= 2048 * 1.2]
    near_one = [s for s in L.sizes if 4096 <= s <= 4096 * 1.1]
    assert len(near_half) >= 3 and len(near_one) >= 3


def test_pick_smallest_bucket_that_holds_the_item():
    L = BucketLadder(4096, 8192)
    for n in range(1, 8193, 37):
        b = L.pick(n)
        if b is None:
            continue
        assert b >= n and b in L.sizes
        assert all(s < n for s in L.sizes if s < b)     # no smaller bucket holds it
        assert b <= n * L.max_padding_ratio


def test_eager_fallback_beyond_padding_ratio_and_ceiling():
    L = BucketLadder(4096, 8192, max_padding_ratio=1.25)
    assert L.pick(100) is None          # 2048 / 100 pads far beyond 1.25
    assert L.pick(2048) == 2048
    assert L.pick(1700) == 2048         # 2048 / 1700 = 1.20 <= 1.25
    assert L.pick(1600) is None         # 2048 / 1600 = 1.28 > 1.25
    L2 = BucketLadder(4096, 8192, max_padding_ratio=1.5)
    assert L2.pick(1600) == 2048
    assert L.pick(8192) == 8192 and L.pick(8193) is None and L.pick(0) is None


def test_pick_ratio_boundary_exact():
    L = BucketLadder(1000, 2000, factors=(1.0, 2.0), align=1, max_padding_ratio=1.25)
    assert L.sizes == [1000, 2000]
    assert L.pick(800) == 1000          # 1000 / 800 = 1.25: allowed
    assert L.pick(799) is None          # 1000 / 799 > 1.25
    assert L.pick(1001) is None         # 2000 / 1001 > 1.25
    assert L.pick(1600) == 2000


def test_capture_order_largest_first():
    L = BucketLadder(4096, 8192)
    assert L.capture_order() == sorted(L.sizes, reverse=True)


@pytest.mark.parametrize("args", [(0, 10), (10, 0), (10, 10, DEFAULT_FACTORS, 0)])
def test_ladder_rejects_bad_arguments(args):
    with pytest.raises(ValueError):
        BucketLadder(*args)

"""Grouping schedule (host logic): which denoising steps run k-means, and
the amortised prepare cost.  The MarkTechPost abstract (yifor post on
VC-Attention) states that grouping runs only in the first 25% of the
denoising steps and that a permutation is reused across 4 adjacent steps."""
import pytest

from bit_attention_video_smooth_amd.schedule import GroupingSchedule


def test_forty_steps_group_three_times():
    s = GroupingSchedule(40)
    assert s.grouping_window == 10
    assert s.grouping_steps() == [0, 4, 8]
    # every step reuses the permutation of the latest grouping step
    latest = [max(g for g in s.grouping_steps() if g <= t) for t in range(40)]
    assert latest[:4] == [0] * 4 and latest[4:8] == [4] * 4 and set(latest[8:]) == {8}


@pytest.mark.parametrize("n,frac,reuse,expect", [
    (10, 0.25, 4, [0]),            # window ceil(2.5) = 3
    (16, 0.25, 4, [0]),            # window 4
    (17, 0.25, 4, [0, 4]),         # window 5
    (8, 1.0, 1, list(range(8))),   # group every step
    (8, 0.0, 4, [0]),              # never regroup after the first step
    (1, 0.25, 4, [0]),
])
def test_grouping_steps(n, frac, reuse, expect):
    assert GroupingSchedule(n, frac, reuse).grouping_steps() == expect


def test_amortised_prepare_cost():
    s = GroupingSchedule(40)
    assert s.amortised(10.0, 2.0) == pytest.approx((3 * 10.0 + 37 * 2.0) / 40)


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        GroupingSchedule(0)
    with pytest.raises(ValueError):
        GroupingSchedule(10, 1.5)
    with pytest.raises(ValueError):
        GroupingSchedule(10, 0.25, 0)
    with pytest.raises(ValueError):
        GroupingSchedule(10).regroup(10)

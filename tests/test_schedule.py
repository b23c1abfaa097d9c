"""Host logic of the selection-reuse schedule (video_diffusion_block_amd/schedule.py)."""
import pytest

from video_diffusion_block_amd.schedule import refresh_steps


def test_every_one_recomputes_every_step():
    assert refresh_steps(10, 1) == [True] * 10


def test_middle_segment_reuses_between_refreshes():
    # 20 steps: middle [ceil(3), ceil(17)) = [3, 17); every 4 -> 3, 7, 11, 15 refresh,
    # 16 reuses, 17.. are past the middle
    plan = refresh_steps(20, 4)
    assert [s for s, r in enumerate(plan) if r] == [0, 1, 2, 3, 7, 11, 15, 17, 18, 19]


def test_whole_schedule_as_middle():
    plan = refresh_steps(9, 3, middle=(0.0, 1.0))
    assert plan == [True, False, False, True, False, False, True, False, False]


def test_empty_middle_recomputes_everything():
    assert refresh_steps(7, 5, middle=(0.5, 0.5)) == [True] * 7


def test_fraction_of_refreshes_in_a_50_step_schedule():
    plan = refresh_steps(50, 3)
    # 8 steps before the middle, 8 from step 43 on, and 12 of the 35 middle steps
    assert sum(plan) == 8 + 7 + 12


@pytest.mark.parametrize("args", [(0, 1), (10, 0), (10, 2, (0.6, 0.4)), (10, 2, (-0.1, 0.5))])
def test_rejects_bad_arguments(args):
    with pytest.raises(ValueError):
        refresh_steps(*args)

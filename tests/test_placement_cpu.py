"""The placement search's decisions, on the host: which trial sets it keeps,
when it stops, and that it hands back the kept set.  The allocation and the
timing are replaced by stand-ins; the GPU test covers the real ones."""
import pytest
import torch

from sharded_mixed_precision_step_amd import placement

pytestmark = pytest.mark.cpu


class Clock:
    def __init__(self, step=1.0):
        self.t, self.step = 0.0, step

    def __call__(self):
        self.t += self.step
        return self.t


def _run(times, *, trials=10, budget_s=1e9, min_gain=0.005, fail_at=None, clock=None):
    """Search over CPU tensors.  times[0] is the first set's time, times[k]
    trial k's; fail_at: the trial whose allocation fails."""
    first = [torch.arange(5, dtype=torch.float32) + i for i in range(3)]
    made, released, seq = [], [0], iter(times)

    def make_set(cur):
        if fail_at is not None and len(made) + 1 == fail_at:
            return None
        new = [t.clone() for t in cur]
        made.append(new)
        return new

    def release():
        released[0] += 1

    res = placement._search(first, lambda s: next(seq), make_set, release, trials=trials,
                            budget_s=budget_s, min_gain=min_gain,
                            clock=clock or Clock())
    return first, made, released[0], res


def test_keeps_only_trials_that_beat_the_kept_set_by_the_margin():
    first, made, released, (best, initial, final, done, kept) = _run(
        [10.0, 11.0, 9.0, 8.99, 8.0, 7.97], trials=5)
    # 9.0 beats 10 by 10 %; 8.99 is within 0.5 % of 9.0; 8.0 beats 9.0;
    # 7.97 is within 0.5 % of 8.0
    assert kept == [2, 4] and done == 5
    assert initial == 10.0 and final == 8.0
    assert best is made[3]
    assert released == 5
    for a, b in zip(best, first):
        assert torch.equal(a, b)


def test_nothing_better_returns_the_first_set():
    first, made, _, (best, initial, final, done, kept) = _run([5.0, 6.0, 5.0, 7.0], trials=3)
    assert kept == [] and done == 3 and best is first and final == initial == 5.0


def test_stops_at_the_first_failed_allocation():
    first, made, released, (best, _, final, done, kept) = _run(
        [10.0, 9.0, 8.0, 7.0], trials=10, fail_at=3)
    assert done == 2 and kept == [1, 2] and final == 8.0 and best is made[1]
    assert released == 3          # after each trial, and after the failure


def test_stops_when_the_budget_is_spent():
    # the clock advances 1 s per reading: the start reads 1, the checks
    # before trials 1..4 read 2..5 (1..4 s elapsed), the fifth check 6 (5 s)
    _, _, _, (_, _, _, done, _) = _run([10.0] * 20, trials=20, budget_s=4.5, clock=Clock())
    assert done == 4


def test_zero_trials_times_the_first_set_only():
    first, made, released, (best, initial, final, done, kept) = _run([4.0], trials=0)
    assert done == 0 and made == [] and released == 0 and best is first and final == 4.0

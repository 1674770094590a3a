"""Host logic of bench.py that needs no GPU: the untimed prewarm runs the
step in batches of ten, synchronising after each, until its time has
passed, and a zero prewarm runs nothing."""
import os
import sys
import time

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


class FakeTorch:
    """Counts synchronisations; stands in for torch in bench.prewarm."""

    class cuda:
        syncs = 0

        @classmethod
        def synchronize(cls):
            cls.syncs += 1


def test_prewarm_runs_batches_until_its_time_has_passed():
    calls = []

    def step():
        calls.append(time.perf_counter())
        time.sleep(0.001)

    FakeTorch.cuda.syncs = 0
    t0 = time.perf_counter()
    n = bench.prewarm(FakeTorch, step, 30.0)
    elapsed = (time.perf_counter() - t0) * 1e3
    assert n == len(calls) and n % 10 == 0 and n >= 10
    assert FakeTorch.cuda.syncs == n // 10
    assert elapsed >= 30.0
    # it stops at the first batch boundary past its time
    assert (calls[-10] - t0) * 1e3 < 30.0 + 5.0


def test_zero_prewarm_runs_nothing():
    FakeTorch.cuda.syncs = 0
    assert bench.prewarm(FakeTorch, lambda: None, 0.0) == 0
    assert FakeTorch.cuda.syncs == 0

"""CPU tests of the GPU tests' hang guard (tests/hang_guard.py): the drain
returns once the stream is idle and calls the exit hook on timeout; the
watchdog fires only when the body overruns."""
import time

from tests import hang_guard


class FakeClock:
    def __init__(self):
        self.t = 0.0

    def __call__(self):
        return self.t

    def sleep(self, dt):
        self.t += dt


def test_drain_returns_when_the_stream_goes_idle():
    clock = FakeClock()
    answers = iter([False, False, False, True])
    fired = []
    ok = hang_guard.drain(lambda: next(answers), 10.0, lambda: fired.append(1), poll_s=0.5,
                          clock=clock, sleep=clock.sleep)
    assert ok and not fired and clock.t == 1.5


def test_drain_calls_the_exit_hook_when_the_stream_never_finishes():
    clock = FakeClock()
    fired = []
    ok = hang_guard.drain(lambda: False, 20.0, lambda: fired.append(clock.t), poll_s=1.0,
                          clock=clock, sleep=clock.sleep)
    assert not ok and fired == [20.0]


def test_watchdog_fires_only_on_overrun():
    fired = []
    dog = hang_guard.Watchdog(5.0, lambda: fired.append(1))
    assert dog.stop() is False and not fired
    dog = hang_guard.Watchdog(0.05, lambda: fired.append(1))
    time.sleep(0.3)
    assert dog.stop() is True and fired == [1]

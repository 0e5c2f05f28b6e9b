"""Hang guard of the GPU tests.

A test whose kernels never finish would otherwise stall the suite until an
outer time limit kills it, with nothing printed about which case hung.  Two
host-side checks bound every GPU test instead:

* a watchdog thread: if the test body has not returned within
  ``body_limit_s``, it prints the test's id and ends the process with
  ``EXIT_HANG`` (``os._exit``: no re-exec, no kernel kill; the main thread
  may be blocked inside a device synchronisation, which only the process's
  end releases);
* a drain after the body: the test's stream is polled with
  ``hipStreamQuery`` (``torch.cuda.Stream.query``) until its work is done,
  for at most ``drain_limit_s``, with the same exit on timeout -- so work a
  test left queued cannot hang the next one.

The waiting logic takes the query and the exit as arguments, so CPU tests
drive it with a fake stream and a recorded exit.
"""
import os
import sys
import threading
import time

EXIT_HANG = 3


def report_and_exit(nodeid: str, what: str, limit_s: float) -> None:
    sys.stdout.flush()
    sys.stderr.write(f"\n[hang-guard] {nodeid}: {what} did not finish within {limit_s:.0f} s; "
                     f"ending the process (exit {EXIT_HANG})\n")
    sys.stderr.flush()
    os._exit(EXIT_HANG)


def drain(query, limit_s: float, on_timeout, poll_s: float = 1e-3,
          clock=time.monotonic, sleep=time.sleep) -> bool:
    """Poll ``query()`` until it returns True (True) or ``limit_s`` has passed
    (calls ``on_timeout()``, returns False)."""
    deadline = clock() + limit_s
    while not query():
        if clock() >= deadline:
            on_timeout()
            return False
        sleep(poll_s)
    return True


class Watchdog:
    """Calls ``on_timeout()`` from a daemon thread unless ``stop()`` comes
    within ``limit_s``."""

    def __init__(self, limit_s: float, on_timeout):
        self._done = threading.Event()
        self._fired = False

        def run():
            if not self._done.wait(limit_s):
                self._fired = True
                on_timeout()

        self._thread = threading.Thread(target=run, name="gpu-hang-guard", daemon=True)
        self._thread.start()

    def stop(self) -> bool:
        """Disarm; True if the watchdog had already fired."""
        self._done.set()
        self._thread.join(timeout=5.0)
        return self._fired

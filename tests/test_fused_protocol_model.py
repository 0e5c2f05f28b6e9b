"""CPU model of the fused last-split-done merge (tests/protocol/
last_split_done_model.cpp): threads in random arrival order, empty splits,
counters reused across calls.  Built with ThreadSanitizer, the protocol as
the decode kernel runs it must pass with no race reported; each planted
mistake (counting in before the state is stored, no counter reset, empty
splits that do not count in) must fail."""
import os
import shutil
import subprocess

import pytest

SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "protocol",
                   "last_split_done_model.cpp")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("protocol") / "last_split_done_model")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread", SRC,
                    "-o", exe], check=True, capture_output=True, text=True)
    return exe


def run(exe, mode, seed, calls=12, threads=8):
    env = dict(os.environ, TSAN_OPTIONS="exitcode=66 halt_on_error=1 report_signal_unsafe=0")
    return subprocess.run([exe, mode, str(seed), str(calls), str(threads)], env=env,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_protocol_merges_once_in_split_order_without_races(model, seed):
    r = run(model, "correct", seed)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "WARNING: ThreadSanitizer" not in r.stderr
    assert "0 failed group checks" in r.stdout


@pytest.mark.parametrize("mode", ["signal_early", "no_reset", "skip_empty"])
def test_planted_mistakes_are_caught(model, mode):
    r = run(model, mode, 5)
    # signal_early: a data race (ThreadSanitizer, exit 66) or a wrong merge;
    # the others: a group that merges zero times or leaves its counter set
    assert r.returncode in (1, 66), (mode, r.returncode, r.stdout, r.stderr[-2000:])

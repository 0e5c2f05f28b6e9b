"""The per-wave timeline of the diagnostics build (libspa_timeline.so):
bench.py --timeline runs in a child process (this process has loaded
libspa.so) on a small page-split shape with the fused merge and on the
ragged int8 batch (head-grouped producer), and every step a wave reached is
stamped no earlier than the step before it."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
@pytest.mark.parametrize("config", [1, 5])
def test_timeline_steps_are_ordered(config):
    print(f"[case] timeline config {config}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", str(config),
                        "--timeline", "--timeline-calls", "2", "--warmup", "20",
                        "--settle-ms", "0"], capture_output=True, text=True, timeout=110,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    assert rec["library"] == "libspa_timeline.so"
    assert rec["waves"] > 0 and all(0 < x < 10000 for x in rec["span_us"])
    assert rec["links"], rec
    for name, d in rec["links"].items():
        assert d["min_us"] >= 0, (name, d)
    steps = [rec["step_median_us"][k] for k in ("entry", "length known", "pages done", "end")]
    assert steps == sorted(steps)
    if config == 1:   # small page-split grid: the fused merge runs in the producer launch
        assert "merge done" in rec["step_median_us"]

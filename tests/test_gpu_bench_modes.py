"""bench.py's optional launch modes run and print their bench line: one
launch for layout + dispatch, timed as replays of a captured graph, on the
128 x 1024 top-2 workload (a few steps)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_one_launch_graph_mode():
    r = subprocess.run([sys.executable, "bench.py", "--workload", "tiny_128x1024_e16_top2", "--steps", "5",
                        "--warmup", "2", "--cpu-seconds", "0", "--cold-reps", "1", "--one-launch", "--graph"],
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    rec = json.loads(line)
    assert rec["launch"] == "graph replay, layout and dispatch in one launch"
    assert rec["value"] > 0 and rec["steps"] == 5

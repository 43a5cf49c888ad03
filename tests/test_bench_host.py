"""Host logic of bench.py (no GPU): the one-GPU contract, the algorithmic work
that the roofline is priced on, and the rule that a stored traffic figure is
reported only for the solver sources it was measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


@pytest.mark.parametrize("m,n", [(1, 1), (1, 5), (4, 1), (3, 4), (6, 5)])
def test_solver_flops_counts_every_feedback_pair(m, n):
    # FastKron page, section 2.2: an entry's error reaches every later entry of
    # its row (through N_A) and of its column (through N_B), one multiply-add each
    pairs = 0
    for i in range(m):
        for j in range(n):
            for i2 in range(m):
                for j2 in range(n):
                    if (i2 == i and j2 > j) or (j2 == j and i2 > i):
                        pairs += 1
    assert bench.solver_flops(m, n) == 2 * pairs


def test_traffic_only_for_the_measured_sources(monkeypatch):
    t = bench.solver_traffic(4096, 4096)
    if t is not None:
        assert 1e8 < t < 1e11
    assert bench.solver_traffic(1024, 4096) is None
    # any other source text gives another hash: the stored figure is then withheld
    monkeypatch.setattr(bench, "SOLVER_SOURCES", bench.SOLVER_SOURCES + ("bench.py",))
    assert bench.solver_traffic(4096, 4096) is None

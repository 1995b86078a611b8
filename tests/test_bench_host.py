"""Host logic of bench.py (CPU only): the one-GPU guard and the grouping of
consecutive steps into captured graphs."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_steps_per_graph_divides_both_counts():
    assert bench.steps_per_graph(256, 32) == 16
    assert bench.steps_per_graph(48, 16) == 16
    assert bench.steps_per_graph(200, 20) == 4
    assert bench.steps_per_graph(7, 0) == 1
    for k in range(1, 70):
        for w in range(0, 40):
            g = bench.steps_per_graph(k, w)
            assert k % g == 0 and w % g == 0 and 1 <= g <= 16


def test_graph_plan_replays_every_step_in_phase_order():
    for P in range(1, 9):
        for g in range(1, 17):
            plan = bench.graph_plan(P, g)
            # replaying the graphs in turn, for several cycles, runs phase i % P at step i
            steps = [k for _ in range(3) for graph in plan for k in graph]
            assert steps == [i % P for i in range(len(steps))], (P, g)
            assert all(len(graph) == g for graph in plan)

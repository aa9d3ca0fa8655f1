"""bench.py's command line on the CPU: the help text, and the refusal of more
than one GPU (the lookup is measured on one GPU's share of the table)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_help_lists_the_workloads():
    r = run("--help")
    assert r.returncode == 0
    for word in ("--steps", "--warmup", "--gpus", "gpu_d512", "host_d512", "--graph", "--batch-scan", "--flushed",
                 "--sharded", "--encode"):
        assert word in r.stdout


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_sharded_leg_refuses_a_shard_count_out_of_range():
    r = run("--sharded", "65", "--steps", "1", "--warmup", "0")
    assert r.returncode in (1, 2)  # 2: refused; 1 on a machine without a GPU, which is checked first
    assert r.stdout.strip() == ""

"""bench.py's command-line contract, checked on the CPU: it measures one GPU only, so any
other GPU count, or a launch under a multi-rank launcher, ends with exit status 2 and a
message before any device work; nonsensical step counts end the same way."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    if env_extra:
        env.update(env_extra)
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("gpus", ["2", "8", "0"])
def test_other_gpu_counts_are_refused(gpus):
    r = run_bench(["--gpus", gpus])
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_multi_rank_launch_is_refused():
    r = run_bench(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    assert "one GPU only" in r.stderr


@pytest.mark.parametrize("args", [["--steps", "0"], ["--warmup", "-1"]])
def test_bad_step_counts_are_refused(args):
    r = run_bench(args)
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    assert "--steps must be >= 1" in r.stderr

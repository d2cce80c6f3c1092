"""bench.py's command line without a GPU: it measures one GPU only and says
so for any other --gpus, or for a multi-rank launch, with exit code 2."""
import os
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]


def run(args, env=None):
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_multi_rank_launch_is_refused():
    r = run([], env=dict(os.environ, WORLD_SIZE="2"))
    assert r.returncode == 2
    assert "multi-rank" in r.stderr

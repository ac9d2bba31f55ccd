"""Command-line contract of bench.py that holds without a GPU: it measures one GPU and
refuses any other count, and it refuses to run (rather than fall back to the CPU) when
no ROCm device is present."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*argv, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                          cwd=ROOT, env=e, capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("argv,env", [(("--gpus", "2"), None),
                                      (("--gpus", "8", "--steps", "1"), None),
                                      ((), {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = _run(*argv, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line is printed for a refused run


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the behaviour without a GPU")
def test_no_gpu_is_refused_not_run_on_the_cpu():
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "needs a ROCm GPU" in r.stderr
    assert r.stdout.strip() == ""

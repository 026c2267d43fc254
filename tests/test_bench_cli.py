"""Host-side checks of bench.py's command line (no GPU needed).

The measurement itself runs on the GPU; these pin the contract around it:
one GPU only (any other count exits with a message before touching a
device), the documented options exist, and a machine without a GPU gets an
error instead of a number.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args, env=None, timeout=120):
    e = dict(os.environ)
    if env:
        e.update(env)
    return subprocess.run([sys.executable, BENCH, *args], cwd=ROOT, env=e, capture_output=True, text=True,
                          timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""                     # no JSON line for a run that did not happen


def test_world_size_above_one_is_refused():
    r = _run(env={"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_options_of_the_contract_exist():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--settle-ms", "--config", "--mode", "--no-cpu-baseline"):
        assert opt in r.stdout, opt


def test_without_a_gpu_there_is_no_number():
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this case is about machines without one")
    r = _run("--no-cpu-baseline", "--steps", "1", "--warmup", "0", "--settle-ms", "0")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""

"""bench.py's command-line contract, checked on the CPU: more than one GPU is
refused with a message, and without a GPU it exits non-zero before timing."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args, env=None):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          timeout=300, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = run(env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_help_lists_the_contract_flags():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout


def test_without_a_gpu_it_fails_loudly():
    import torch
    if torch.cuda.is_available():
        return
    r = run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert "needs a GPU" in r.stderr and r.stdout == ""

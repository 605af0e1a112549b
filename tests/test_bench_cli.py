"""bench.py's contract on the host: more than one GPU is refused with a message (the library
has no multi-GPU path; the bench measures one GPU); the help text lists the workload options."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--alignment", "--route-groups", "--fp8", "--backward", "--eager", "--bf16-partials"):
        assert opt in r.stdout

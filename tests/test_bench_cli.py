"""The benchmark's command-line contract on the CPU: more than one GPU is
refused with a message (the step runs on one GPU; nothing is launched), and
the flags parse."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = run("--gpus", n)
        assert r.returncode == 2, r
        assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_legs():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--workload", "--zero2", "--offload", "--amp", "--composed", "--cpu-sample",
                 "--no-skipped-leg"):
        assert flag in r.stdout, flag

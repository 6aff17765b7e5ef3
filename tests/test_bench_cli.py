"""bench.py's command line on a host without a GPU: more than one GPU is refused with a message
before anything touches a device, and the help text lists the flags."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _run("--gpus", n)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr and r.stdout == ""


def test_help_lists_the_flags():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--dtype", "--no-cpu-baseline", "--no-chunk", "--no-extra"):
        assert flag in r.stdout, flag

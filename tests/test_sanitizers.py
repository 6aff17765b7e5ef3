"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only): the ABI validators
and their fuzz, the expert-record header checks (every single-bit flip, truncations, bad offsets) and
the oracle with its pins run in a subprocess against builds instrumented by tests/sanitize_build.py
(sanitizers on the host side of librvq.so, on the oracle and on the input generator).  Any
sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

import sanitize_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_abi_cpu.py", "tests/test_oracle_pins.py", "tests/test_quant_checks.py"]


@pytest.fixture(scope="module")
def outdir():
    try:
        sanitize_build.asan_runtime()
    except (FileNotFoundError, subprocess.CalledProcessError, OSError) as e:
        pytest.skip(f"no clang sanitizer runtime: {e}")
    return sanitize_build.build()


def test_host_code_is_clean_under_asan_and_ubsan(outdir):
    env = sanitize_build.runtime_env(outdir)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + SUITES,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    line = [l for l in out.splitlines() if l.startswith("sanitized builds mapped:")]
    assert line and all(n in line[0] for n in ("librvq.so", "liboracle_san.so", "libsynth_san.so")), out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]

"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

The pin tests and the mutant tests run again in a child process that loads
the sanitized build of the oracle (``ORACLE_SANITIZE=1``, gcc's ASan runtime
preloaded; any sanitizer report ends that process with an error), so every
array access the pins and the planted mistakes make is bounds-checked.  A
planted one-past-the-end read shows that the sanitizer is live.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN = obuild.asan_runtime()

pytestmark = pytest.mark.skipif(ASAN is None, reason="gcc's ASan runtime is not installed")


def _env():
    env = dict(os.environ)
    env.update(LD_PRELOAD=ASAN,
               ASAN_OPTIONS="detect_leaks=0",  # the Python interpreter's own allocations
               UBSAN_OPTIONS="print_stacktrace=1",
               ORACLE_SANITIZE="1",
               OMP_NUM_THREADS="2")
    return env


def test_pins_and_mutants_under_sanitizers():
    obuild.build(sanitize=True)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-n", "4",
           "-m", "not gpu", "tests/test_oracle_pins.py", "tests/test_oracle_mutants.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=_env(), capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out


def test_sanitizer_reports_a_planted_overflow(tmp_path):
    """Read one element past the end of the score buffer (the last causal row
    has as many visible keys as the buffer holds): ASan must stop the run."""
    src = open(obuild.SRC).read()
    old = "double m = scores[0];"
    assert src.count(old) == 1
    path_c = tmp_path / "overflow.c"
    path_c.write_text(src.replace(old, "double m = scores[n];"))
    lib = tmp_path / "liboverflow.so"
    subprocess.run(["gcc"] + obuild.cflags(sanitize=True, opt="-O1")
                   + ["-w", "-o", str(lib), str(path_c), "-lm"], check=True)
    script = (
        "import numpy as np, oracle\n"
        "rng = np.random.default_rng(0)\n"
        "x = rng.standard_normal((1, 8, 1, 16)).astype(np.float16)\n"
        f"oracle.Oracle({str(lib)!r}).prefill(x, x, x, True)\n"
        "print('finished')\n")
    r = subprocess.run([sys.executable, "-c", script], cwd=ROOT, env=_env(),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
    assert "finished" not in r.stdout

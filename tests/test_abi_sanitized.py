"""The C-ABI library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): libattn.so is rebuilt with the host
side instrumented (device code unchanged), and the ABI tests -- argument
validation of every entry point, status strings, exported symbols -- run
against that build in a child process with clang's ASan runtime preloaded.
Any sanitizer report ends the child with an error.  No GPU is touched: every
call the ABI tests make is rejected on the host or needs no device."""
import os
import subprocess
import sys

import pytest

from attention_attn_prefill_amd import build as abuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN = abuild.asan_runtime()

pytestmark = pytest.mark.skipif(ASAN is None, reason="clang's ASan runtime is not installed")


@pytest.mark.timeout(900)
def test_abi_tests_under_host_sanitizers(tmp_path):
    lib = str(tmp_path / "libattn_host_sanitized.so")
    abuild.build(host_sanitize=True, out=lib, jobs=8)
    script = (
        "import sys\n"
        "from attention_attn_prefill_amd import binding\n"
        f"binding.LIB_PATH = {lib!r}\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu',\n"
        "                      'tests/test_abi.py']))\n")
    env = dict(os.environ)
    env.update(LD_PRELOAD=ASAN, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", script], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out

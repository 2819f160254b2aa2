"""The C-ABI host tests again, against a build whose host code carries AddressSanitizer and
UndefinedBehaviorSanitizer (device code unchanged; see build_sanitized.py).  Runs on the CPU: the
host tests never launch a kernel.  A sanitizer report ends the child process with a failure."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_suite_under_asan_and_ubsan():
    from full_spatiotemporal_attention_amd import build_sanitized as bs
    try:
        bs.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = bs.build()
    assert os.path.exists(lib)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_cabi_host.py"),
                        "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=bs.sanitizer_env(), stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    out = r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out

"""The CPU tests of the C ABI (tests/test_host.py) once more against the host
library compiled with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
(kie_api.cpp alone; no device code).  Any out-of-bounds access, use after
free or undefined behaviour in the argument checks, the packer or the
schedule validator aborts the child process."""
import os
import subprocess
import sys

import pytest

from decode_persistent_monokernel_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_under_address_and_ub_sanitizers():
    try:
        B.build_host_sanitized()
    except RuntimeError as e:  # pragma: no cover - toolchain without sanitizers
        pytest.skip(f"sanitizer build unavailable: {e}")
    env = B.sanitizer_env()
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail

"""The C ABI's host code (argument checks, workspace plans, launch sequencing)
under AddressSanitizer, on the CPU: the ABI tests run again in a child process
against a variant of the library whose host code is built with ASan, with the
sanitizer runtime preloaded.  A heap or stack overrun in the validation code
fails the child."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_checks_under_address_sanitizer():
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    sys.path.insert(0, ROOT)
    from block_text_diffusion_amd import build
    lib = build.build_asan()
    env = dict(os.environ, DG_LIBRARY=lib, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout

"""The ABI validation tests (tests/test_abi.py) run again against a build of
the C ABI layer with AddressSanitizer and UndefinedBehaviorSanitizer (host
code only; the kernels are the release objects). Any out-of-bounds access,
use of freed memory, signed overflow, misaligned access or other undefined
behaviour on the host paths the tests drive aborts the run."""
import os
import subprocess
import sys

import pytest
import torch

from exact_io_aware_29_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(torch.cuda.device_count() > 0,
                    reason="the ABI checks it reruns use fake pointers: GPU-less hosts only")
def test_abi_suite_under_asan_and_ubsan():
    lib = B.SANITIZED_OUT
    if not os.path.exists(lib):
        if B.build_sanitized() is None:
            pytest.skip("g++ or the sanitizer runtime is not available")
    env = dict(os.environ)
    env.update(FA_LIBRARY=lib, LD_PRELOAD=B.ASAN_RUNTIME,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = subprocess.run([sys.executable, "-c",
                            "from exact_io_aware_29_amd import _abi; print(_abi.load()._name)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out and "failed" not in out

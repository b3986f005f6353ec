"""The argument checks of every C entry point under host AddressSanitizer and
UndefinedBehaviorSanitizer: the fake-pointer validation cases of test_abi.py run
in a child process against libfa built with host-only sanitizers
(io_aware_exact_16_amd.build.build_asan), with the sanitizer runtime preloaded.
CPU only: no kernel is launched (with a GPU visible the validation cases skip)."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT, gpu_available


@pytest.mark.skipif(gpu_available(), reason="the fake-pointer validation cases run only where no GPU is visible")
def test_validation_cases_clean_under_host_asan():
    sys.path.insert(0, ROOT)
    from io_aware_exact_16_amd.build import asan_runtime, build_asan
    lib = build_asan()
    env = dict(os.environ, LD_PRELOAD=asan_runtime(), FA_ABI_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), "-k", "validation or status or exports"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout

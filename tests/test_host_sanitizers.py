"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
the library is built again with instrumented host code (device code as usual)
and the host-only ABI and binding tests run against it in a child process
with the sanitizer runtime preloaded. Any report fails the run (halt on the
first error). Nothing here launches a kernel."""
import os
import subprocess
import sys

import pytest

from mixture_experts_ffn_align_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no shared AddressSanitizer runtime next to the compiler")
    out = str(tmp_path_factory.mktemp("san") / "libmoe_ffn.so")
    build.build_host_sanitized(out)
    env = dict(os.environ, MOE_FFN_LIBRARY=out, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return out, env


def test_the_child_loads_the_instrumented_library(sanitized):
    out, env = sanitized
    code = ("import mixture_experts_ffn_align_amd._binding as B; B.lib(); "
            "print(any(l.rstrip().endswith(B.LIB_PATH) for l in open('/proc/self/maps')))")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0 and res.stdout.strip() == "True", res.stdout + res.stderr[-2000:]


def test_abi_validation_under_sanitizers(sanitized):
    _, env = sanitized
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                          "tests/test_abi.py", "tests/test_binding_checks.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    text = res.stdout[-3000:] + res.stderr[-3000:]
    assert res.returncode == 0, text
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error:" not in res.stderr, text
    assert " passed" in res.stdout, text

"""The CPU suite once more under AddressSanitizer and UndefinedBehaviorSanitizer:
the oracle and the library's host code (argument validation, launch set-up)
are rebuilt with both sanitizers (``make sanitize``), and the CPU tests run
in a child process that preloads the sanitizer runtime and loads those
builds.  Any finding ends the child with an error."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.sanitize


def _asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.skip("no clang AddressSanitizer runtime in this image")
    return hits[-1]


def test_cpu_suite_clean_under_asan_and_ubsan():
    rt = _asan_runtime()
    jobs = str(min(8, os.cpu_count() or 1))
    for d in ("oracle", os.path.join("mxfp4_activation_quantizer_amd", "csrc")):
        subprocess.run(["make", "-j", jobs, "-C", os.path.join(ROOT, d), "sanitize"], check=True,
                       stdout=subprocess.DEVNULL)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "KQ_TEST_SANITIZED_LIBS": "1",
        # the interpreter and the libraries it loads are not instrumented
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0:"
                        "verify_asan_link_order=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu and not sanitize", os.path.join(ROOT, "tests")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "error" not in r.stdout.lower().split("passed")[-1], tail

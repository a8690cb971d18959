"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds libsvg2 with both sanitizers on the host side (build_sanitized.py) and
runs the CPU ABI tests (test_abi_cpu.py: every entry point's argument
validation, size queries and status strings, plus the binding's buffer checks)
in a child process that loads that build, with clang's ASan runtime
preloaded.  Any sanitizer report fails the run (halt_on_error)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed for the sanitized build")
def test_abi_under_host_asan_ubsan():
    from sparse_attention_video_head_amd import build_sanitized as S
    lib = S.build()
    # the build is instrumented: its host code calls the ASan and UBSan runtimes
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, LD_PRELOAD=S.asan_runtime(), SVG2_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out

"""The C ABI's host-side checks (tests/test_abi.py: symbol exports, the wave
scheduler, argument validation and its error paths) rerun against a build of
the runtime's host code with AddressSanitizer and UndefinedBehaviorSanitizer
(long_context_recurrent_amd.build.build_host_sanitized), in a child process
with the sanitizer runtime preloaded.  A memory error or undefined behaviour
on any of those paths ends the child with a sanitizer report.  CPU only."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def test_abi_checks_under_host_sanitizers():
    from long_context_recurrent_amd import build as B
    lib = B.build_host_sanitized()
    rt = B.asan_runtime()
    assert os.path.exists(rt), rt
    # the sanitized build really carries the instrumentation
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm
    env = dict(os.environ, LD_PRELOAD=rt, ARMT_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    check = ("import sys; sys.path.insert(0, %r)\n"
             "from long_context_recurrent_amd import armt as A\n"
             "A.load_library()\n"
             "maps = open('/proc/self/maps').read()\n"
             "assert A.library_path() in maps and 'libclang_rt.asan' in maps\n" % ROOT)
    p = subprocess.run([sys.executable, "-c", check], env=env, capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stdout + p.stderr
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = p.stdout + p.stderr
    assert p.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]

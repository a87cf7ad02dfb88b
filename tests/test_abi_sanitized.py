"""The C-ABI checks of tests/test_abi.py again, against a copy of the library
whose host code (argument validation, workspace carving, launch sequences) is
built with AddressSanitizer and UndefinedBehaviorSanitizer.  CPU only: every
call fails validation (or finds no GPU) before a kernel runs.  The check builds
the sanitized copy, runs the ABI tests in a child process with the ASan runtime
preloaded, and confirms that the child really loaded the instrumented library."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = [pytest.mark.slow,
              pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                 reason="hipcc not available")]


def test_abi_under_address_and_ub_sanitizers():
    from compressive_memory_transformer_amd import build as b
    lib = b.build(sanitize=True)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms, "library not instrumented"
    env = dict(os.environ)
    env.update(LD_PRELOAD=b.sanitizer_runtime(), INFINI_ATTN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = ("import sys; sys.path.insert(0, %r); from compressive_memory_transformer_amd import infini as ia; "
             "ia.load_library(); maps = open('/proc/self/maps').read(); "
             "assert ia.LIB_PATH in maps and 'libclang_rt.asan' in maps; print('sanitized library loaded')" % ROOT)
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr

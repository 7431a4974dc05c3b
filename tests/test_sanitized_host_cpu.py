"""The C ABI's host code (argument validation, extent, overlap and overflow
arithmetic, dispatch) under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

Builds libfa.so with -fsanitize=address,undefined in its host code
(``exact_io_aware_02_amd.build.build_sanitized``; device code as usual),
checks that the build is instrumented, and runs the ABI and binding tests
against it in a child process with the ASan runtime preloaded.  Any ASan
report or UBSan runtime error fails the run (halt_on_error).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def test_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    from exact_io_aware_02_amd import build

    lib = build.build_sanitized(str(tmp_path / "libfa_sanitized.so"))
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms, "host code is not ASan-instrumented"
    assert "__ubsan_handle" in syms, "host code is not UBSan-instrumented"
    env = build.sanitizer_env(lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        os.path.join(ROOT, "tests", "test_binding_checks_cpu.py")],
                       env=env, cwd=str(tmp_path), capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout

"""The host code of the C ABI under AddressSanitizer and UndefinedBehavior-
Sanitizer.  The sanitized code is the validation, workspace planning, table
building and launch preparation that runs before any kernel.

The library is built from the same sources with the sanitizers on its host
side only (``build.build(sanitize=True)``; device code unchanged).  The CPU
tests of ``tests/test_abi.py`` then run against it in a child process that
preloads the ASan runtime.  Those tests call every exported entry point, with
valid descriptors and with each kind of invalid one.  Any out-of-bounds
access, use after free, overflow or other undefined behaviour in that code
ends the child with a report.  Leak checking is off: the Python interpreter
itself does not free everything at exit."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.timeout(900)
def test_abi_tests_pass_with_host_sanitizers(tmp_path):
    rt = _asan_runtime()
    if rt is None or not (os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc")):
        pytest.skip("hipcc or the ASan runtime is not available")
    from nf4_bit_quantized_amd import build
    lib = build.build(out_path=str(tmp_path / "libqlora_nf4_sanitized.so"), sanitize=True)
    env = dict(os.environ,
               LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               QLORA_NF4_LIBRARY=lib)
    probe = ("import nf4_bit_quantized_amd as q, ctypes; q.lib(); "
             "assert q.LIB_PATH == %r; ctypes.CDLL(None).__asan_report_load1; print('sanitized library loaded')" % lib)
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "sanitized library loaded" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=800)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr

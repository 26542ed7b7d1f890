"""The C-ABI checks of tests/test_abi_cpu.py once more, against a build of
the library whose host code is compiled with AddressSanitizer (device code
unchanged): every host-side validation path the CPU tests reach runs under
ASan, which aborts on an out-of-bounds or use-after-free access.  Builds the
variant (hipcc cross-compiles without a GPU) and runs the tests in a child
Python with the sanitizer runtime preloaded."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow


def test_abi_checks_under_host_asan():
    from linear_complexity_video_mate_amd import build

    lib = build.build(asan=True)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms, "the variant is not instrumented"
    env = dict(os.environ, LD_PRELOAD=build.asan_runtime(), LINGEN_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout

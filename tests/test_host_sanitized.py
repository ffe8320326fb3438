"""The library's host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

flce_api.hip (argument checks, workspace layouts, the chunk loops, the
allocation-free entry point's scratch lookup) is compiled for the CPU by g++
with both sanitizers, against stand-in HIP headers and stub launchers
(tests/host_sanitize/): no kernel runs; each stub launch checks that the
memory its kernel would touch lies inside the caller's buffers.  In child
processes with the sanitizer runtime preloaded:
  * every case of tests/test_abi_host.py runs against that library;
  * tests/host_sanitize/sweep_paths.py makes successful calls of every entry
    point over tiny, ragged and full-size shapes and counts out-of-buffer
    ranges.
Any sanitizer report aborts the child (halt_on_error) and fails the test.
No GPU is needed.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "host_sanitize")
CXX = shutil.which("g++")


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    if CXX is None:
        pytest.skip("g++ not available")
    asan = subprocess.run([CXX, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("the AddressSanitizer runtime is not installed")
    out = str(tmp_path_factory.mktemp("san") / "libflce_host_san.so")
    csrc = os.path.join(ROOT, "linear_cross_entropy_06_amd", "csrc")
    cmd = [CXX, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-Wall", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", SAN, "-I", os.path.join(ROOT, "include"),
           "-I", csrc, "-x", "c++", os.path.join(csrc, "flce_api.hip"),
           "-x", "c++", os.path.join(SAN, "stub_runtime.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out, asan


def _run(san, code):
    lib, asan = san
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", code.replace("@LIB@", lib)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    report = (r.stdout + r.stderr)[-6000:]
    assert r.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report
    return report


def test_abi_host_cases_under_sanitizers(san_lib):
    out = _run(san_lib, (
        "import sys\n"
        "import linear_cross_entropy_06_amd._lib as L\n"
        "L.LIB_PATH = '@LIB@'\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi_host.py']))\n"))
    assert " passed" in out and " failed" not in out, out


def test_every_entry_point_stays_inside_its_buffers(san_lib):
    out = _run(san_lib, (
        "import sys\n"
        "sys.path.insert(0, 'tests/host_sanitize')\n"
        "import sweep_paths\n"
        "sys.exit(sweep_paths.main('@LIB@'))\n"))
    assert "successful calls checked" in out and "FAIL" not in out, out

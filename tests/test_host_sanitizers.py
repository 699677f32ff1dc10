"""Host AddressSanitizer / UndefinedBehaviorSanitizer builds of the planner
(convolution_nhwc_conv2d_amd/csrc/select.cpp) and of the oracle, driven with a
seeded mix of valid, extreme and invalid arguments (tests/sanitize/*_driver.cpp).
Both are plain C++ with no GPU code; g++ builds them here, in a temporary
directory."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


def _build_and_run(sources, includes, tmp):
    exe = os.path.join(tmp, "driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-pthread"] + SAN + [f"-I{i}" for i in includes] + sources + ["-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # verify_asan_link_order=0: whatever the environment preloads stays loaded, ahead of the ASan runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


def test_select_under_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        out = _build_and_run(
            [os.path.join(ROOT, "convolution_nhwc_conv2d_amd", "csrc", "select.cpp"),
             os.path.join(HERE, "select_driver.cpp")],
            [os.path.join(ROOT, "include"), os.path.join(ROOT, "convolution_nhwc_conv2d_amd", "csrc")], tmp)
    assert "select ok" in out


def test_oracle_under_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        out = _build_and_run([os.path.join(ROOT, "oracle", "oracle.cpp"), os.path.join(HERE, "oracle_driver.cpp")],
                             [], tmp)
    assert "oracle ok" in out

"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
library's codebook construction (csrc/codebook.cpp) and the oracle's C coder
(oracle/coder.c), built with gcc/g++ -fsanitize=address,undefined (no
recovery: the first report aborts) together with sanitize_driver.cpp, which
drives both over edge cases, random inputs, invalid arguments and corrupted
streams.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def test_host_code_under_asan_and_ubsan(tmp_path):
    gcc, gxx = shutil.which("gcc"), shutil.which("g++")
    if not gcc or not gxx:
        pytest.skip("no host C/C++ compiler")
    coder_o = str(tmp_path / "coder.o")
    drv = str(tmp_path / "sanitize_driver")
    subprocess.run([gcc, "-std=c11", "-pthread"] + FLAGS + ["-c", os.path.join(ROOT, "oracle", "coder.c"),
                    "-o", coder_o], check=True)
    subprocess.run([gxx, "-std=c++17", "-pthread"] + FLAGS + [
        "-I", os.path.join(ROOT, "include"),
        os.path.join(ROOT, "static_codebook_lossless_amd", "csrc", "codebook.cpp"),
        os.path.join(ROOT, "tests", "sanitize_driver.cpp"), coder_o, "-o", drv], check=True)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "halt_on_error=1:detect_leaks=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([drv], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "all checks passed" in r.stdout

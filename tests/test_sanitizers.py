"""The packer (csrc/tq_host.cpp) and the C oracle built with AddressSanitizer
and UndefinedBehaviorSanitizer (host code only), exercised by
sanitize_driver.py in a child process."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="no host compiler")
def test_host_code_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    host = str(tmp_path / "libtq_host_san.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", *SAN,
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "binary_g128_bit_amd", "csrc"),
                    os.path.join(ROOT, "binary_g128_bit_amd", "csrc", "tq_host.cpp"), "-o", host],
                   check=True)
    orc = oracle.build(str(tmp_path / "liboracle_san.so"), extra_flags=SAN)
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan + " " + ubsan
    # the interpreter itself is not built for leak checking
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize_driver.py"), host, orc],
                       capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert "clean" in r.stdout

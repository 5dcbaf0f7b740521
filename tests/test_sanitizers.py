"""The host half of the library (dfh_host.cpp) and the CPU oracle (oracle.c)
built with AddressSanitizer and UndefinedBehaviorSanitizer (g++ and gcc, host
code only) and run through tests/sanitize/driver.cpp: every host entry point
on edge-size inputs of all kinds, sections against the oracle's, oracle
decodes of the library's containers, file round trips and damaged files.
CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="no host compiler")
def test_host_library_and_oracle_under_asan_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    objs = []
    o = str(tmp_path / "oracle.o")
    subprocess.check_call(["gcc", "-std=c99", "-pthread"] + SAN +
                          ["-c", os.path.join(ROOT, "oracle", "oracle.c"), "-o", o])
    objs.append(o)
    for src in (os.path.join(ROOT, "lossless_entropy_coded_huffman_amd", "csrc", "dfh_host.cpp"),
                os.path.join(HERE, "driver.cpp")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.check_call(["g++", "-std=c++17", "-pthread"] + SAN + inc + ["-c", src, "-o", o])
        objs.append(o)
    exe = str(tmp_path / "driver")
    subprocess.check_call(["g++", "-pthread"] + SAN + objs + ["-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, str(tmp_path / "c.dfc")], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-6000:]
    assert "sanitize driver: ok" in r.stdout

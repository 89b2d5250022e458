"""The host C++ of libsx under AddressSanitizer and UBSan (CPU only).

api.cpp (argument checks, workspace sizing, the token-class and realign
planners) and seg_index.cpp (the segment index: SHA-256 block hash, block
pool, virtual entries, eviction) are built with g++ and
-fsanitize=address,undefined together with tests/host_asan_driver.cpp, which
runs the planners on random batches, the segment index through random
operation sequences, and the argument checks of every device entry point
(whose launchers are stubs that abort if reached).  Any sanitizer report or
failed check fails the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "segment_level_kv_amd", "csrc")
ROCM = "/opt/rocm"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_host_code_under_address_sanitizer(tmp_path):
    flags = ["-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-I" + os.path.join(ROCM, "include")]
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "seg_index.cpp"),
                os.path.join(ROOT, "tests", "host_asan_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run(["g++", *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    exe = str(tmp_path / "host_driver")
    lib = os.path.join(ROCM, "lib")
    r = subprocess.run(["g++", "-fsanitize=address,undefined", *objs, "-L" + lib, "-Wl,-rpath," + lib,
                        "-lamdhip64", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "all checks passed" in out

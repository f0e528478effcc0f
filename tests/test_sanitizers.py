"""The host library and the oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/exercise.cpp drives the host encoder (ecf8_host.cpp,
ecf8v_host.cpp) and the oracle (oracle/*.c) with exact-size buffers over
edge sizes, skewed and uniform inputs and four (C, TB) shapes, checking the
library against the oracle byte for byte.  This test builds it with g++
-fsanitize=address,undefined (host code only: no HIP source is compiled
here) and requires a clean run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_library_and_oracle_under_sanitizers(tmp_path):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if not gxx or not gcc:
        pytest.skip("no host compiler")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
    inc = ["-I" + os.path.join(ROOT, "include")]
    objs = []
    for src in ("oracle/ecf8_oracle.c", "oracle/ecf8v_oracle.c"):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.check_call([gcc, "-std=c99", "-c", os.path.join(ROOT, src), "-o", o] + san)
        objs.append(o)
    for src in ("lossless_entropy_coded_ecf8_amd/csrc/ecf8_host.cpp", "lossless_entropy_coded_ecf8_amd/csrc/ecf8v_host.cpp",
                "tests/sanitize/exercise.cpp"):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.check_call([gxx, "-std=c++17", "-c", os.path.join(ROOT, src), "-o", o] + inc + san)
        objs.append(o)
    exe = str(tmp_path / "exercise")
    subprocess.check_call([gxx, "-o", exe] + objs + san + ["-lpthread"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert " 0 failures" in r.stdout

"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed): tests/asan/host_checks.cpp runs the host Lloyd-Max solver over
a range of dimensions and widths and every entry point's synchronous argument
checks with invalid arguments, linked against the library's sources built with
the sanitizers on their host code (the device code is compiled as usual and
never runs)."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_vector_06_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_host_code_under_asan_and_ubsan(tmp_path):
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC] + SAN
    jobs = [[HIPCC, "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + common
            + ["-c", os.path.join(CSRC, f"{n}.hip"), "-o", str(tmp_path / f"{n}.o")]
            for n in ("tq_encode", "tq_decode", "tq_probe")]
    jobs += [[HIPCC] + common + ["-x", "c++", "-c", src, "-o", str(tmp_path / obj)]
             for src, obj in ((os.path.join(CSRC, "tq_codebook.cpp"), "cb.o"),
                              (os.path.join(ROOT, "tests", "asan", "host_checks.cpp"), "main.o"))]
    with ThreadPoolExecutor(4) as ex:
        for r in ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), jobs):
            assert r.returncode == 0, r.stdout + r.stderr
    exe = str(tmp_path / "host_checks")
    objs = [str(tmp_path / o) for o in ("main.o", "cb.o", "tq_encode.o", "tq_decode.o", "tq_probe.o")]
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address,undefined"] + objs
                       + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "host checks passed" in r.stdout, r.stdout + r.stderr

"""The CPU oracle and the library's host validation path under AddressSanitizer
and UndefinedBehaviorSanitizer (CPU only; no device call is made).

Every HIP source is compiled with the sanitizers on its host side only
(`-Xarch_host`, so device code is built as usual), the oracle and a small C++
driver (tests/native/sanitize_driver.cpp) with the same clang, and the
program is linked against the HIP runtime.  The driver runs the oracle on
seeded small inputs and calls every entry point with malformed arguments,
expecting the documented status before any device call.  Any sanitizer
report ends the program with a non-zero status.
"""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
from paged_block_scoring_amd.build import SOURCES as HIP_SOURCES  # the library's own source list
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="needs hipcc and ROCm clang")
def test_oracle_and_host_validation_under_sanitizers():
    tmp = tempfile.mkdtemp(prefix="qsa_san_")
    try:
        inc = ["-I", os.path.join(ROOT, "include")]
        jobs = []
        objs = []
        for src in HIP_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            jobs.append([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + HOST_SAN + inc +
                        ["-c", os.path.join(ROOT, "paged_block_scoring_amd", "csrc", src), "-o", obj])
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
        obj = os.path.join(tmp, "oracle.o")
        objs.append(obj)
        jobs.append([CLANG, "-std=c11", "-ffp-contract=off", "-pthread"] + san +
                    ["-c", os.path.join(ROOT, "oracle", "qsa_oracle.c"), "-o", obj])
        obj = os.path.join(tmp, "driver.o")
        objs.append(obj)
        jobs.append([CLANGXX, "-std=c++17"] + san + inc +
                    ["-c", os.path.join(ROOT, "tests", "native", "sanitize_driver.cpp"), "-o", obj])
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), jobs))
        for cmd, r in zip(jobs, results):
            assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
        exe = os.path.join(tmp, "sanitize_driver")
        link = [CLANGXX] + san + ["-pthread", "-o", exe] + objs + [
            "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm"]
        r = subprocess.run(link, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(link)}\n{r.stdout}\n{r.stderr}"
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, f"sanitized run failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
        assert "sanitized host checks passed" in r.stdout
    finally:
        shutil.rmtree(tmp, ignore_errors=True)

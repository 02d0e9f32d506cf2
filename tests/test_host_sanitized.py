"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of libosx.so is compiled with the sanitizers on its host side
only (the gfx950 device code is compiled as usual), linked with the native
self-test ``tests/native/abi_selftest.cpp`` into one executable, and run.  The
self-test sweeps the planners over ordinary and extreme shapes and drives every
entry point into each of its argument checks; a heap or stack overrun, a signed
overflow, a bad shift or a leak in that host code ends the run with a sanitizer
report.  No kernel is launched, so no GPU is needed.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "online_softmax_02_amd", "csrc")
OUT = os.path.join(ROOT, "online_softmax_02_amd", "_build", "host_sanitized")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

# Sanitizers for the host side of each hipcc compile only: every -fsanitize
# option is preceded by -Xarch_host.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
# The self-test and the final link are host-only clang++ steps.
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _sources():
    import importlib.util
    spec = importlib.util.spec_from_file_location("_osx_build", os.path.join(ROOT, "online_softmax_02_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b.SOURCES, b.ARCH


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not found")
def test_host_code_under_asan_and_ubsan():
    sources, arch = _sources()
    os.makedirs(OUT, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, f"--offload-arch={arch}", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
        _run(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, sources))
    test_obj = os.path.join(OUT, "abi_selftest.o")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "native", "abi_selftest.cpp"), "-o", test_obj])
    exe = os.path.join(OUT, "abi_selftest")
    _run([CLANGXX, *SAN, test_obj, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])

    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    print(r.stdout)
    assert r.returncode == 0, f"sanitized self-test failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-6000:]}"
    assert "0 failures" in r.stdout
    shutil.rmtree(OUT, ignore_errors=True)

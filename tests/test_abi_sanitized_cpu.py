"""The C ABI's host-side argument checks under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): api.hip is rebuilt with the sanitizers on its host code only, linked with the
kernels' objects of the normal build, and the host-side test files run against that library
in a child process with the sanitizer runtime preloaded.  Any report (out-of-bounds access,
signed overflow, invalid shift, ...) ends the child with a non-zero status."""

import glob
import os
import subprocess
import sys

import pytest

from fp8_quantized_gemm_amax_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_abi_cpu.py", "tests/test_gemm_plan_cpu.py", "tests/test_binding_outputs_cpu.py"]


def asan_runtime():
    for pattern in ("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                    "/opt/rocm*/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(pattern))
        if hits:
            return hits[-1]
    return None


def test_abi_checks_clean_under_host_sanitizers(tmp_path):
    rt = asan_runtime()
    objs = [os.path.join(build.OBJ_DIR, s.replace(".hip", ".o")) for s in build.SOURCES if s != "api.hip"]
    if rt is None or not all(os.path.exists(o) for o in objs):
        pytest.skip("no sanitizer runtime, or the library has not been built")
    # sanitizers on the host pass only: -Xarch_host right before each option
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = [f for f in build.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    api_o = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libfp8amax_san.so")
    cc = build.hipcc()
    subprocess.run([cc, *flags, *san, "-shared-libasan", "-I", build.INCLUDE, "-I", build.CSRC, "-c", "-o", api_o,
                    os.path.join(build.CSRC, "api.hip")], check=True, capture_output=True, timeout=600)
    subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-shared-libasan", "-o", lib, api_o, *objs],
                   check=True, capture_output=True, timeout=600)
    env = dict(os.environ, FP8AMAX_LIBRARY=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: a sanitizer report goes straight to stderr before the process ends
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu", *HOST_TESTS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout

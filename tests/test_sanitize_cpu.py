"""Host code under the address and undefined-behaviour sanitizers (CPU only).

Two programs are built in a temporary directory and run; each must exit 0
with no sanitizer report:

* the oracle's C integer GEMM (oracle/int_gemm.c), built with gcc
  -fsanitize=address,undefined, driven by tests/sanitize/oracle_gemm_check.c
  (brute force on ragged shapes, the all-127 closed form, the int32 bound and
  its first wrapping K, cancelling signs);
* the library's host code (the C-ABI validation in csrc/w8a8_api.hip and the
  plan choice and launch set-up in the other sources), built with hipcc with
  the sanitizers on the host side only (-Xarch_host before each
  -fsanitize=; the device code is compiled as usual), driven by
  tests/sanitize/abi_check.cpp, which repeats the validation checks of
  test_abi_cpu.py through the C ABI and runs the plan choice over a grid of
  shapes.  Nothing launches: no GPU is needed.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w8a8_int8_quantized_token_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def _clean(out: str) -> bool:
    return "runtime error" not in out and "ERROR: AddressSanitizer" not in out \
        and "ERROR: LeakSanitizer" not in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_gemm_sanitized(tmp_path):
    exe = str(tmp_path / "oracle_check")
    rc, out = _run(["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Werror",
                    "-o", exe, os.path.join(SAN, "oracle_gemm_check.c"),
                    os.path.join(ROOT, "oracle", "int_gemm.c")])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV)
    assert rc == 0 and _clean(out), out
    assert "oracle gemm checks ok" in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_host_code_sanitized(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
             "-I", os.path.join(ROOT, "include")]
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_w8a8_build", os.path.join(ROOT, "w8a8_int8_quantized_token_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    srcs = [os.path.join(CSRC, f) for f in build.SOURCES]   # every source of the library
    srcs.append(os.path.join(SAN, "abi_check.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        return obj, _run([HIPCC, *flags, "-c", src, "-o", obj])

    with ThreadPoolExecutor(len(srcs)) as ex:
        results = list(ex.map(compile_one, srcs))
    for obj, (rc, out) in results:
        assert rc == 0, out
    exe = str(tmp_path / "abi_check")
    rc, out = _run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, "-o", exe, *[o for o, _ in results]])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV)
    assert rc == 0 and _clean(out), out
    assert "abi host checks ok" in out

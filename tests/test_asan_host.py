"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds gqa_api.hip's host code (no device code: the kernels are replaced by
stand-ins that report "no device") with both sanitizers, links it with
tests/asan/abi_host_driver.cpp, and runs the driver. The driver checks argument
validation, planning over a grid of shapes up to the 32-bit limits, the error
paths of the prepare / launch / append entry points and the per-thread error
message; any out-of-bounds access, use after free or undefined behaviour
(signed overflow, bad shifts, misaligned access) in that code aborts it.
Runs on the CPU; needs hipcc and ROCm's clang.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "gqa_kv_cache_attn_amd", "csrc")
ASAN_DIR = os.path.join(ROOT, "tests", "asan")

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc / ROCm clang not found")
    out = tmp_path_factory.mktemp("asan")
    api_o, stubs_o, drv_o, exe = (str(out / n) for n in ("api.o", "stubs.o", "driver.o", "driver"))
    # Host side only: each sanitizer flag goes to the host compilation.
    host_san = [x for flag in SAN for x in ("-Xarch_host", flag)]
    _run([HIPCC, "--offload-arch=gfx950", "--offload-host-only", "-O1", "-g", "-std=c++20", "-fPIC",
          *host_san, "-Wno-unused-command-line-argument", "-I", INCLUDE,
          "-c", os.path.join(CSRC, "gqa_api.hip"), "-o", api_o])
    common = [CLANG, "-std=c++20", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
              "-I", CSRC, "-I", os.path.join(ROCM, "include")]
    _run([*common, "-c", os.path.join(ASAN_DIR, "kernel_stubs.cpp"), "-o", stubs_o])
    _run([*common, "-c", os.path.join(ASAN_DIR, "abi_host_driver.cpp"), "-o", drv_o])
    _run([CLANG, *SAN, api_o, stubs_o, drv_o, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    return exe


def test_the_build_is_instrumented(driver):
    nm = shutil.which("nm") or os.path.join(ROCM, "llvm", "bin", "llvm-nm")
    syms = _run([nm, driver]).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms


def test_abi_host_code_is_clean_under_asan_and_ubsan(driver):
    env = dict(os.environ)
    # The HIP runtime's own allocations outlive main; leaks are not checked.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([driver], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0 and "ALL OK" in res.stdout, res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in res.stderr
    assert "runtime error" not in res.stderr

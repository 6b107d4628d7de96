"""The C-ABI layer's host code under AddressSanitizer and
UndefinedBehaviorSanitizer: api.hip is compiled with both (host side only:
each -fsanitize= goes after -Xarch_host, the device pass is untouched), the
kernel launchers are replaced by stubs that abort if reached, and a C driver
(tests/abi_sanitize_driver.c) makes calls that validation must reject: NULL,
out-of-range and overflowing shapes, invalid decays, misaligned and
overlapping pointers, short workspaces. The driver's decay array is exactly
`heads` doubles of heap memory, so a check that reads past it is reported.
CPU only: no call reaches the GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "retnet_retention_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HERE = os.path.dirname(os.path.abspath(__file__))
ROCM = "/opt/rocm"
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.timeout(600)
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    if not (os.path.exists(hipcc) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm toolchain not found")
    api_o, stubs_o, drv_o, exe = (str(tmp_path / n) for n in ("api.o", "stubs.o", "driver.o", "driver"))
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    _run([hipcc, *common, *SAN_HOST, "-c", os.path.join(CSRC, "api.hip"), "-o", api_o])
    _run([CLANGXX, "-x", "hip", "--cuda-host-only", "-D__HIP_PLATFORM_AMD__", "-O1", "-g", "-std=c++17", "-fPIC",
          "-I", INCLUDE, "-I", CSRC, "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-c", os.path.join(HERE, "abi_sanitize_stubs.cpp"), "-o", stubs_o])
    _run([CLANG, "-O1", "-g", "-I", INCLUDE, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-c", os.path.join(HERE, "abi_sanitize_driver.c"), "-o", drv_o])
    _run([CLANGXX, "-fsanitize=address,undefined", drv_o, api_o, stubs_o, "-o", exe,
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr

"""AddressSanitizer and UndefinedBehaviorSanitizer builds, on the CPU.

- The C oracles with tests/sanitize/oracle_checks.c (gcc): strided inputs,
  T across the 256-token checkpoint blocks, split invariance, T = 0 and
  refused dimensions.
- The C ABI's argument validation with tests/sanitize/abi_checks.c: api.hip
  built with its host code instrumented (hipcc, the sanitizer flags given to
  the host pass only), linked against launcher stubs that abort, so the run
  needs no GPU and would stop at any launch.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(SAN, "oracle_checks.c"), os.path.join(ROOT, "oracle", "linrec_oracle.c"),
          os.path.join(ROOT, "oracle", "deltarule_oracle.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "oracle checks passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="hipcc not found")
def test_abi_validation_under_asan_ubsan(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "state_passing_amd", "csrc")]
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    api_o, stub_o, drv_o = (str(tmp_path / n) for n in ("api.o", "stubs.o", "abi_checks.o"))
    _run([hipcc, "-std=c++17", "-O1", "-g", "--offload-arch=gfx950", "-fno-omit-frame-pointer",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, *inc,
          "-c", os.path.join(ROOT, "state_passing_amd", "csrc", "api.hip"), "-o", api_o])
    # plain C++ (no device code) for the stubs and the driver
    _run([clang + "++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", *inc, "-I", os.path.join(ROCM, "include"),
          "-c", os.path.join(SAN, "launch_stubs.cpp"), "-o", stub_o])
    _run([clang, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          *inc, "-c", os.path.join(SAN, "abi_checks.c"), "-o", drv_o])
    exe = str(tmp_path / "abi_checks")
    _run([clang + "++", "-fsanitize=address,undefined", drv_o, api_o, stub_o,
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
          "-o", exe])
    # the HIP runtime's own allocations at load time are not this library's
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=0")
    r = _run([exe], env=env, timeout=300)
    assert "abi checks passed" in r.stdout

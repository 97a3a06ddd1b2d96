"""CPU sanitizer runs (no GPU): the oracle under AddressSanitizer + UndefinedBehaviorSanitizer and
under ThreadSanitizer (its pthread pool), and the C ABI's host code (api.cpp: argument checks,
dispatch, error text) under AddressSanitizer + UndefinedBehaviorSanitizer with the device launchers
and HIP runtime calls stubbed. Each builds a small driver from tests/sanitize/ with the host
compilers (gcc, g++) and runs it: it must exit 0 and print no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


def _build_and_run(tmp_path, cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"build failed:\n{r.stdout}\n{r.stderr}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer", "ERROR: LeakSanitizer"):
        assert marker not in out, out
    assert "all checks passed" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = tmp_path / "orc_asan"
    _build_and_run(tmp_path, ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
                              "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", str(exe),
                              os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_driver.c"),
                              "-lm", "-pthread"], exe)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_thread_pool_under_thread_sanitizer(tmp_path):
    exe = tmp_path / "orc_tsan"
    _build_and_run(tmp_path, ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fsanitize=thread", "-o",
                              str(exe), os.path.join(ROOT, "oracle", "oracle.c"),
                              os.path.join(SAN, "oracle_driver.c"), "-lm", "-pthread"], exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_c_abi_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = tmp_path / "api_asan"
    csrc = os.path.join(ROOT, "quantized_matmul_mlx_amd", "csrc")
    _build_and_run(tmp_path, ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                              "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
                              "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + csrc, "-o", str(exe),
                              os.path.join(csrc, "api.cpp"), os.path.join(SAN, "api_driver.cpp")], exe)

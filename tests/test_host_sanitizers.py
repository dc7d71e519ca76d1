"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only).

The C-ABI's host logic (pkv_api.cpp, with the device launchers replaced by
stubs that are never reached) and the oracle's C core are built with both
sanitizers and driven through every call that needs no device: the drivers
exit non-zero on a failed check, the sanitizers on any memory or undefined-
behaviour error.  Device code is checked on the GPU by determinism and
parity tests instead (no device sanitizer is used).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "long_context_decode_pkv_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, cwd, env=None, timeout=600):
    r = subprocess.run(cmd, cwd=cwd, env=env, capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not installed")
def test_c_abi_host_logic_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    cmd = [CLANG, "-std=c++17", "-w", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *SAN,
           os.path.join(CSRC, "pkv_api.cpp"), os.path.join(HERE, "sanitize", "device_stubs.cpp"),
           os.path.join(HERE, "sanitize", "host_driver.cpp"),
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe]
    _run(cmd, str(tmp_path))
    r = _run([exe], str(tmp_path), env=ENV)
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_core_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-fopenmp", *SAN, os.path.join(ROOT, "oracle", "pkv_oracle.c"),
          os.path.join(HERE, "sanitize", "oracle_driver.c"), "-lm", "-o", exe], str(tmp_path))
    r = _run([exe], str(tmp_path), env=dict(ENV, OMP_NUM_THREADS="4"))
    assert "all checks passed" in r.stdout
